"""Helpers shared by the GPU tests: device transfer of stored synthetic inputs, running the four C-ABI
calls, and comparing their outputs with the float64 oracle."""

from __future__ import annotations

import ctypes
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402
from oracle import gptq_ref as ref  # noqa: E402

PROBES_LIB = os.path.join(ROOT, "tests", "libgptq_probes.so")

TAU = 1e-3          # tie window, in units of the rounding ratio
SCALE_RTOL = 1e-5   # scales and zero points
LOSS_RTOL = 1e-3    # layer reconstruction error


def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def dev_tensor(a: np.ndarray, dtype: str):
    torch = torch_cuda()
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to("cuda:0")


def params_of(case, **kw):
    import post_weight_quantization_20_amd as g
    d = dict(bits=case.bits, group_size=case.group_size, block_size=case.block_size, act_order=case.act_order,
             damp=case.damp)
    d.update(kw)
    return g.Params(**d)


def gpu_layer(case, W=None, chunks=None, params=None):
    """Runs the four calls on a synthetic case; returns numpy outputs."""
    torch = torch_cuda()
    import post_weight_quantization_20_amd as g
    W = synth.weight(case) if W is None else W
    chunks = [synth.x_chunk(case, c) for c in range(case.n_chunks)] if chunks is None else chunks
    params = params_of(case) if params is None else params
    Wd = dev_tensor(W, case.w_dtype)
    Xd = [dev_tensor(x, case.x_dtype) for x in chunks]
    res = g.quantize_layer(Wd, Xd, params)
    torch.cuda.synchronize()
    out = dict(H=res.H.cpu().numpy(), U=res.U.cpu().numpy(), perm=res.perm.cpu().numpy().astype(np.int64),
               codes=res.quant.codes.cpu().numpy(), scales=res.quant.scales.cpu().numpy(),
               zeros=res.quant.zeros.cpu().numpy(), g_idx=res.quant.g_idx.cpu().numpy(),
               loss=float(res.quant.loss.cpu().numpy()[0]),
               packed=None if res.packed is None else res.packed.cpu().numpy())
    return W, chunks, out


def dequant(codes, scales, zeros, g_idx):
    """Q[r][c] = scale[r][g_idx[c]] * (code[r][c] - zero[r][g_idx[c]])."""
    s = scales.astype(np.float64)[:, g_idx]
    z = zeros.astype(np.float64)[:, g_idx]
    return s * (codes.astype(np.float64) - z)


def check_quant_parity(gpu, o_quant, codes_tol=0.001):
    """Parity of the column loop's outputs with an oracle run that followed the GPU at ties.

    o_quant: the oracle's QuantResult run with follow=(gpu codes in processing order, gpu zeros).
    Requires: no code or zero differs outside tie windows; adopted-and-different decisions are at
    most `codes_tol` of all codes; scales within 1e-5 relative; loss within 1e-3 relative.
    """
    codes = gpu["codes"]
    assert np.array_equal(gpu["g_idx"], o_quant.g_idx)
    mism = int(np.count_nonzero(codes != o_quant.codes))
    assert mism == 0, f"{mism} of {codes.size} codes differ outside tie windows"
    assert np.array_equal(gpu["zeros"], o_quant.zeros), "zero points differ outside tie windows"
    assert o_quant.adopted_diff <= codes_tol * codes.size, (o_quant.adopted_diff, codes.size)
    s = gpu["scales"].astype(np.float64)
    rel = np.abs(s - o_quant.scales) / np.abs(o_quant.scales)
    assert float(np.max(rel)) <= SCALE_RTOL, float(np.max(rel))
    assert abs(gpu["loss"] - o_quant.loss) <= LOSS_RTOL * abs(o_quant.loss), (gpu["loss"], o_quant.loss)


FACTOR_VS_LAPACK = 10.0   # factor error allowed, in units of float32 LAPACK's error on the same matrix


def lapack_f32_factor(Hh: np.ndarray) -> np.ndarray:
    """The upper Cholesky factor of Hh^-1 computed by LAPACK in float32 along the sketch's literal
    route (potrf, potri, potrf): what float32 arithmetic achieves on this matrix."""
    from scipy.linalg import lapack
    L, info = lapack.spotrf(Hh.astype(np.float32), lower=1)
    assert info == 0
    Ai, info = lapack.spotri(L, lower=1)
    assert info == 0
    Ai = np.tril(Ai) + np.tril(Ai, -1).T
    U, info = lapack.spotrf(Ai, lower=0)
    assert info == 0
    return np.triu(U).astype(np.float64)


def factor_errors(U: np.ndarray, Hh: np.ndarray, Uo: np.ndarray):
    """(max |U - Uo| / max |Uo|, max |U^T U Hh - I|) of a factor U against the float64 oracle's Uo."""
    U = U.astype(np.float64)
    err = float(np.max(np.abs(U - Uo)) / np.max(np.abs(Uo)))
    resid = float(np.max(np.abs(U.T @ U @ Hh - np.eye(Hh.shape[0]))))
    return err, resid


def load_probes():
    if not os.path.exists(PROBES_LIB):
        pytest.skip("probe library not built (run __graft_entry__.build())")
    L = ctypes.CDLL(PROBES_LIB)
    for n in ("probe_mfma_f16", "probe_mfma_bf16", "probe_mfma_f32", "probe_mfma_f32_16", "probe_mfma_f32_4x4",
              "probe_row_bcast", "probe_row_ror15", "probe_div"):
        getattr(L, n).restype = ctypes.c_int
    return L
