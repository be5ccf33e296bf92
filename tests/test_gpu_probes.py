"""Lane layouts of the MFMA builtins, the DPP row broadcast / rotation, and the correctly rounded
division helper, checked on the GPU through a small probe library (tests/gpu_probes.hip)."""

import ctypes

import numpy as np
import pytest

from gpu_util import load_probes, torch_cuda

pytestmark = pytest.mark.gpu


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def test_mfma_f16_bf16_layout():
    torch = torch_cuda()
    L = load_probes()
    rng = np.random.default_rng(1)
    A = rng.integers(-8, 9, size=(32, 16)).astype(np.float32)
    B = rng.integers(-8, 9, size=(16, 32)).astype(np.float32)
    want = A @ B
    for name, tdt in (("probe_mfma_f16", torch.float16), ("probe_mfma_bf16", torch.bfloat16)):
        a = torch.from_numpy(A).to(tdt).view(torch.int16).cuda()
        b = torch.from_numpy(B).to(tdt).view(torch.int16).cuda()
        d = torch.zeros((32, 32), dtype=torch.float32, device="cuda")
        assert getattr(L, name)(_p(a), _p(b), _p(d)) == 0
        assert np.array_equal(d.cpu().numpy(), want), name


def test_mfma_f32_layout():
    torch = torch_cuda()
    L = load_probes()
    rng = np.random.default_rng(2)
    A = rng.integers(-8, 9, size=(32, 2)).astype(np.float32)
    B = rng.integers(-8, 9, size=(2, 32)).astype(np.float32)
    a, b = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    d = torch.zeros((32, 32), dtype=torch.float32, device="cuda")
    assert L.probe_mfma_f32(_p(a), _p(b), _p(d)) == 0
    assert np.array_equal(d.cpu().numpy(), A @ B)


def test_mfma_f32_16x16_layout():
    torch = torch_cuda()
    L = load_probes()
    rng = np.random.default_rng(4)
    A = rng.integers(-8, 9, size=(16, 4)).astype(np.float32)
    B = rng.integers(-8, 9, size=(4, 16)).astype(np.float32)
    a, b = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    d = torch.zeros((16, 16), dtype=torch.float32, device="cuda")
    assert L.probe_mfma_f32_16(_p(a), _p(b), _p(d)) == 0
    assert np.array_equal(d.cpu().numpy(), A @ B)


def test_mfma_f32_4x4_layout():
    torch = torch_cuda()
    L = load_probes()
    rng = np.random.default_rng(5)
    A = rng.integers(-8, 9, size=(4, 4)).astype(np.float32)
    B = rng.integers(-8, 9, size=(4, 64)).astype(np.float32)
    a, b = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
    d = torch.zeros((4, 64), dtype=torch.float32, device="cuda")
    assert L.probe_mfma_f32_4x4(_p(a), _p(b), _p(d)) == 0
    assert np.array_equal(d.cpu().numpy(), A @ B)


def test_row_broadcast_and_rotation():
    torch = torch_cuda()
    L = load_probes()
    x = torch.arange(64, dtype=torch.float32, device="cuda") + 100
    out = torch.zeros(16 * 64, dtype=torch.float32, device="cuda")
    assert L.probe_row_bcast(_p(x), _p(out)) == 0
    got = out.cpu().numpy().reshape(16, 64)
    lanes = np.arange(64)
    for src in range(16):
        assert np.array_equal(got[src], 100 + 16 * (lanes // 16) + src), src
    r = torch.zeros(64, dtype=torch.float32, device="cuda")
    assert L.probe_row_ror15(_p(x), _p(r)) == 0
    assert np.array_equal(r.cpu().numpy(), 100 + 16 * (lanes // 16) + (lanes + 1) % 16)


def test_division_helper_is_correctly_rounded():
    torch = torch_cuda()
    L = load_probes()
    rng = np.random.default_rng(3)
    n = 1 << 22
    s = (10.0 ** rng.uniform(-9, 2, n)).astype(np.float32)
    w = rng.uniform(-30, 30, n).astype(np.float32) * s
    # ratios near half-integers and exact ties, the cases that decide a rounding
    k = n // 4
    m = rng.integers(-40, 40, k).astype(np.float32)
    w[:k] = (m + np.float32(0.5)) * s[:k]
    w[k:2 * k] = np.nextafter(w[k:2 * k], np.float32(np.inf))
    w[:8] = np.float32(0.75)
    s[:8] = np.float32(0.1)
    wd, sd = torch.from_numpy(w).cuda(), torch.from_numpy(s).cuda()
    fast = torch.empty_like(wd)
    ieee = torch.empty_like(wd)
    assert L.probe_div(_p(wd), _p(sd), ctypes.c_int64(n), _p(fast), _p(ieee)) == 0
    f, i = fast.cpu().numpy(), ieee.cpu().numpy()
    assert np.array_equal(f.view(np.uint32), i.view(np.uint32))
    assert np.array_equal(i, w / s)          # the GPU's division equals numpy's float32 division
    assert f[0] == np.float32(7.5)           # 0.75 / 0.1 in float32 (Technical Guide's example)
