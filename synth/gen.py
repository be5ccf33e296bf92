"""Seeded synthetic layer inputs: weights W (rows x d) and calibration activations X (tokens x d).

This module holds random draws and dtype rounding only; it computes no step of the quantization
method. The GPU path and the float64 oracle both consume the stored values it returns, so either
side can regenerate any token chunk on its own.

Recipe (the shapes and distributions stand in for the calibration data and trained layers the
pages use; see the GPTQ tools page, "How it works", Step 1: a few hundred 2,048-token sequences):

* Every draw comes from numpy PCG64 seeded by SeedSequence([2026, *key]); W uses key
  (config, 0, layer); X chunk c of input i uses (config, 1 + i, c); the outlier channel set of
  input i uses (config, 100 + i).
* Values are drawn in float64 and rounded once (round-to-nearest-even) to the storage dtype.
* X is generated per chunk of 2048 tokens (the last chunk of a case may be shorter).
* Outlier channels: round(frac * d) feature indices drawn without replacement; those X columns
  are multiplied by the stated factor before rounding.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace
from typing import Dict, List, Optional, Tuple

import numpy as np

ROOT_SEED = 2026
CHUNK_TOKENS = 2048

DTYPES = ("f32", "f16", "bf16")


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([ROOT_SEED, *[int(k) for k in key]])))


def round_to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values once (nearest-even) to the storage dtype.

    f32 -> float32 array, f16 -> float16 array, bf16 -> uint16 array of bfloat16 bit patterns.
    """
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f32":
        return x.astype(np.float32)
    if dtype == "f16":
        return x.astype(np.float16)
    if dtype == "bf16":
        # Round straight from float64 to 8 significant bits (no float32 double rounding).
        m, e = np.frexp(x)
        r = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)
        bits = r.astype(np.float32).view(np.uint32) >> np.uint32(16)
        return bits.astype(np.uint16)
    raise ValueError(f"unknown dtype {dtype!r}")


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact float64 values of bfloat16 bit patterns."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def to_f64(stored: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of stored inputs."""
    if dtype == "bf16":
        return bf16_bits_to_f64(stored)
    return np.asarray(stored).astype(np.float64)


@dataclass(frozen=True)
class LayerCase:
    """One linear layer's synthetic inputs and quantization settings."""

    name: str
    cfg_id: int
    layer: int           # index of W within the workload (selects the W stream)
    input_id: int        # index of the calibration input (layers sharing X share H)
    rows: int
    d: int
    n: int               # calibration tokens
    w_std: float
    w_dtype: str
    x_dist: str          # "normal" or "laplace"
    x_dtype: str
    outlier_frac: float
    outlier_scale: float
    bits: int = 4
    group_size: int = 128  # <= 0: one group per row
    block_size: int = 128
    act_order: bool = False
    damp: float = 0.01
    chunk: int = CHUNK_TOKENS

    @property
    def n_chunks(self) -> int:
        return (self.n + self.chunk - 1) // self.chunk

    def chunk_tokens(self, c: int) -> int:
        return min(self.chunk, self.n - c * self.chunk)


@dataclass(frozen=True)
class Workload:
    """A named set of layers (one for a single-layer workload, seven for a decoder block)."""

    name: str
    description: str
    layers: Tuple[LayerCase, ...]


def weight(case: LayerCase) -> np.ndarray:
    """W (rows x d) ~ N(0, w_std^2), in the stored dtype."""
    g = _rng(case.cfg_id, 0, case.layer)
    w = g.standard_normal((case.rows, case.d)) * case.w_std
    return round_to_dtype(w, case.w_dtype)


def outlier_channels(case: LayerCase) -> np.ndarray:
    """Sorted feature indices whose activations are scaled by case.outlier_scale."""
    k = int(round(case.outlier_frac * case.d))
    if k <= 0:
        return np.zeros(0, dtype=np.int64)
    g = _rng(case.cfg_id, 100 + case.input_id)
    return np.sort(g.choice(case.d, size=k, replace=False)).astype(np.int64)


def x_chunk(case: LayerCase, c: int, outliers: Optional[np.ndarray] = None) -> np.ndarray:
    """Calibration chunk c: (tokens_c x d) in the stored dtype."""
    t = case.chunk_tokens(c)
    if t <= 0:
        raise IndexError(f"chunk {c} out of range for n={case.n}")
    g = _rng(case.cfg_id, 1 + case.input_id, c)
    if case.x_dist == "normal":
        x = g.standard_normal((t, case.d))
    elif case.x_dist == "laplace":
        x = g.laplace(0.0, 1.0, size=(t, case.d))
    else:
        raise ValueError(case.x_dist)
    if outliers is None:
        outliers = outlier_channels(case)
    if outliers.size:
        x[:, outliers] *= case.outlier_scale
    return round_to_dtype(x, case.x_dtype)


def x_tokens(case: LayerCase, out: Optional[np.ndarray] = None, threads: Optional[int] = None,
             chunks: Optional[List[int]] = None) -> np.ndarray:
    """All (or the listed) chunks stacked into one (tokens x d) array, generated in parallel."""
    idx = list(range(case.n_chunks)) if chunks is None else list(chunks)
    sizes = [case.chunk_tokens(c) for c in idx]
    total = int(sum(sizes))
    np_dt = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[case.x_dtype]
    if out is None:
        out = np.empty((total, case.d), dtype=np_dt)
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    outl = outlier_channels(case)

    def fill(k: int) -> None:
        out[offs[k]:offs[k + 1]] = x_chunk(case, idx[k], outl)

    nthreads = threads or min(16, os.cpu_count() or 1)
    if nthreads <= 1 or len(idx) <= 1:
        for k in range(len(idx)):
            fill(k)
    else:
        with ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(fill, range(len(idx))))
    return out


def make_case(name: str = "case", seed: int = 0, rows: int = 64, d: int = 128, n: int = 512,
              w_std: float = 0.02, w_dtype: str = "f32", x_dist: str = "normal", x_dtype: str = "f32",
              outlier_frac: float = 0.0, outlier_scale: float = 1.0, **quant) -> LayerCase:
    """A free-form case (tests use it for small shapes with the configs' distributions)."""
    return LayerCase(name=name, cfg_id=1000 + seed, layer=0, input_id=0, rows=rows, d=d, n=n,
                     w_std=w_std, w_dtype=w_dtype, x_dist=x_dist, x_dtype=x_dtype,
                     outlier_frac=outlier_frac, outlier_scale=outlier_scale, **quant)


def _c(name, cfg_id, layer, input_id, rows, d, n, **kw) -> LayerCase:
    return LayerCase(name=name, cfg_id=cfg_id, layer=layer, input_id=input_id, rows=rows, d=d, n=n, **kw)


_TOK = 128 * 2048  # 128 sequences of 2048 tokens

_QP = dict(w_std=0.02, w_dtype="f16", x_dist="normal", x_dtype="f16", outlier_frac=0.01, outlier_scale=20.0)
_DP = dict(w_std=0.02, w_dtype="f16", x_dist="laplace", x_dtype="f16", outlier_frac=0.005, outlier_scale=30.0)

CONFIGS: Dict[str, Workload] = {
    "tiny": Workload(
        "tiny", "W 64x128 fp32 N(0,0.02^2); X 512 tokens fp32 N(0,1); 4-bit g32 B32 damp 0.01",
        (_c("tiny", 1, 0, 0, 64, 128, 512, w_std=0.02, w_dtype="f32", x_dist="normal", x_dtype="f32",
            outlier_frac=0.0, outlier_scale=1.0, bits=4, group_size=32, block_size=32, chunk=512),)),
    "q_proj": Workload(
        "q_proj", "Llama-7B q_proj shape: W 4096x4096 fp16; X 262144x4096 fp16 N(0,1), 1% channels x20; "
        "4-bit g128 B128 damp 0.01",
        (_c("q_proj", 2, 0, 0, 4096, 4096, _TOK, bits=4, group_size=128, block_size=128, **_QP),)),
    "down_proj": Workload(
        "down_proj", "Llama-7B down_proj shape: W 4096x11008 fp16; X 262144x11008 fp16 Laplace(0,1), "
        "0.5% channels x30; 4-bit g128 B128 act-order",
        (_c("down_proj", 3, 0, 0, 4096, 11008, _TOK, bits=4, group_size=128, block_size=128,
            act_order=True, **_DP),)),
    "fc2": Workload(
        "fc2", "OPT-175B fc2 shape: W 12288x49152 fp16 N(0,0.01^2); X 131072x49152 fp16 N(0,1), "
        "1% channels x20; 3-bit one group per row, B128",
        (_c("fc2", 4, 0, 0, 12288, 49152, 64 * 2048, w_std=0.01, w_dtype="f16", x_dist="normal",
            x_dtype="f16", outlier_frac=0.01, outlier_scale=20.0, bits=3, group_size=0, block_size=128),)),
}

_BLK = dict(bits=4, group_size=128, block_size=128, act_order=True)
CONFIGS["block"] = Workload(
    "block", "Llama-7B decoder block: q,k,v,o 4096x4096; gate,up 11008x4096; down 4096x11008; fp16 "
    "N(0,0.02^2); inputs attn-in (q,k,v), o-in, mlp-in (gate,up), down-in; 4-bit g128 act-order",
    (
        _c("block.q", 5, 0, 0, 4096, 4096, _TOK, **_QP, **_BLK),
        _c("block.k", 5, 1, 0, 4096, 4096, _TOK, **_QP, **_BLK),
        _c("block.v", 5, 2, 0, 4096, 4096, _TOK, **_QP, **_BLK),
        _c("block.o", 5, 3, 1, 4096, 4096, _TOK, **_QP, **_BLK),
        _c("block.gate", 5, 4, 2, 11008, 4096, _TOK, **_QP, **_BLK),
        _c("block.up", 5, 5, 2, 11008, 4096, _TOK, **_QP, **_BLK),
        _c("block.down", 5, 6, 3, 4096, 11008, _TOK, **_DP, **_BLK),
    ))


def case_from_config(name: str, layer: int = 0, **overrides) -> LayerCase:
    """A layer of a named workload, optionally with fields overridden (e.g. fewer rows or tokens)."""
    c = CONFIGS[name].layers[layer]
    return replace(c, **overrides) if overrides else c


# ------------------------------------------------------------------ stored layers for inference

@dataclass
class StoredLayer:
    """A quantized layer in the stored format: codes uint8 rows x d (original column order),
    scales float32 and zeros int32 rows x ngroups, and g_idx int32 [d] (None: column k in group k // g)."""
    codes: np.ndarray
    scales: np.ndarray
    zeros: np.ndarray
    g_idx: Optional[np.ndarray]
    group_size: int


def stored_layer(seed: int, rows: int, d: int, bits: int = 4, group_size: int = 128, act_order: bool = False,
                 exact: bool = False) -> StoredLayer:
    """Random draws in the stored format, keyed (300, seed).

    codes: uniform over [0, 2^bits). scales: log-uniform in [1e-3, 3e-2], or with exact=True powers of
    two 2^-k, k uniform in 0..3. zeros: uniform over [0, 2^bits), except 5% drawn uniformly from
    [-4, 2^bits + 4) (a group whose weights all share one sign has its zero outside the code range).
    act_order: the groups are g consecutive positions of a uniformly random column order, so g_idx of
    column perm[j] is j // g, the shape the column loop leaves after act-order.
    """
    rng = _rng(300, seed)
    g = d if group_size <= 0 else group_size
    ng = (d + g - 1) // g
    codes = rng.integers(0, 1 << bits, size=(rows, d), dtype=np.uint8)
    if exact:
        scales = np.ldexp(1.0, -rng.integers(0, 4, size=(rows, ng))).astype(np.float32)
    else:
        scales = np.exp(rng.uniform(np.log(1e-3), np.log(3e-2), size=(rows, ng))).astype(np.float32)
    zeros = rng.integers(0, 1 << bits, size=(rows, ng), dtype=np.int64)
    wide = rng.random((rows, ng)) < 0.05
    zeros[wide] = rng.integers(-4, (1 << bits) + 4, size=int(wide.sum()))
    g_idx = None
    if act_order:
        perm = rng.permutation(d)
        g_idx = np.empty(d, dtype=np.int32)
        g_idx[perm] = (np.arange(d) // g).astype(np.int32)
    return StoredLayer(codes=codes, scales=scales, zeros=zeros.astype(np.int32), g_idx=g_idx, group_size=group_size)


def inference_x(seed: int, m: int, d: int, dtype: str = "f16", exact: bool = False) -> np.ndarray:
    """m rows of layer inputs, keyed (301, seed): N(0, 1) rounded to dtype, or with exact=True integers
    uniform in [-2, 2]. Stored as in round_to_dtype."""
    rng = _rng(301, seed)
    x = rng.integers(-2, 3, size=(m, d)).astype(np.float64) if exact else rng.standard_normal((m, d))
    return round_to_dtype(x, dtype)


# ------------------------------------------------------------------ decoder block

@dataclass(frozen=True)
class BlockCase:
    """A synthetic pre-norm decoder block: seven weights (q, k, v, o: hidden x hidden; gate, up:
    inter x hidden; down: hidden x inter) ~ N(0, w_std^2) and a block input X of seqs * seq_len
    tokens ~ N(0, 1) with round(outlier_frac * hidden) channels scaled by outlier_scale (the
    layer configs' attention-input recipe)."""
    hidden: int
    heads: int
    inter: int
    seqs: int
    seq_len: int
    w_std: float = 0.02
    w_dtype: str = "f16"
    x_dtype: str = "f16"
    outlier_frac: float = 0.01
    outlier_scale: float = 20.0


def block_layer_dims(case: BlockCase, i: int) -> Tuple[int, int]:
    """(rows, d) of layer i in the order q, k, v, o, gate, up, down."""
    rows = case.inter if i in (4, 5) else case.hidden
    return rows, (case.inter if i == 6 else case.hidden)


def block_weights(case: BlockCase, seed: int) -> List[np.ndarray]:
    """The seven stored weights, layer i keyed (400, seed, i)."""
    out = []
    for i in range(7):
        rows, d = block_layer_dims(case, i)
        out.append(round_to_dtype(_rng(400, seed, i).standard_normal((rows, d)) * case.w_std, case.w_dtype))
    return out


def block_x(case: BlockCase, seed: int) -> np.ndarray:
    """The stored block input [seqs * seq_len, hidden], keyed (401, seed); outlier channels keyed
    (402, seed)."""
    n = case.seqs * case.seq_len
    k = int(round(case.outlier_frac * case.hidden))
    ch = np.sort(_rng(402, seed).choice(case.hidden, size=k, replace=False))
    x = _rng(401, seed).standard_normal((n, case.hidden))
    x[:, ch] *= case.outlier_scale
    return round_to_dtype(x, case.x_dtype)
