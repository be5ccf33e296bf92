"""Pins of the block oracle (oracle/block_ref.py) against what does not depend on it (CPU only).

* Its pieces against torch's float64 library routines: rms_norm, causal scaled-dot-product
  attention, silu, and the whole forward pass assembled from them (with linear).
* Closed forms: with o and down zero the block is the identity; with q and k zero every query
  weighs the keys equally, so the attention output is the running mean of V within a sequence.
* The driver: stage inputs equal the library forward pass through the weights the pages' order
  prescribes (quantized upstream layers when true-sequential, the original ones otherwise), stage
  0 does not depend on the mode, and the block output runs through all quantized weights.
* Planted mistakes in the oracle's source fail at least one of these checks.
"""

import inspect
import sys
import types

import numpy as np
import pytest

torch = pytest.importorskip("torch")
import torch.nn.functional as F  # noqa: E402

from oracle import block_ref as blk  # noqa: E402
from oracle import gptq_ref as ref  # noqa: E402

SH = blk.BlockShape(hidden=32, heads=2, inter=48, seqs=2, seq_len=40, eps=1e-6)


def _weights(rng, sh, std=0.2):
    dims = [(sh.hidden, sh.hidden)] * 4 + [(sh.inter, sh.hidden)] * 2 + [(sh.hidden, sh.inter)]
    return [rng.standard_normal(d) * std for d in dims]


def _x(rng, sh):
    x = rng.standard_normal((sh.seqs * sh.seq_len, sh.hidden))
    x[:, 3] *= 20.0
    return x


def lib_forward(X, W, sh):
    """The block assembled from torch's own float64 routines."""
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))  # noqa: E731
    X = t(X)
    W = [t(w) for w in W]
    xa = F.rms_norm(X, (sh.hidden,), eps=sh.eps)
    q, k, v = (F.linear(xa, W[i]) for i in range(3))
    dh = sh.hidden // sh.heads

    def heads(a):
        return a.reshape(sh.seqs, sh.seq_len, sh.heads, dh).transpose(1, 2)

    o = F.scaled_dot_product_attention(heads(q), heads(k), heads(v), is_causal=True)
    o_in = o.transpose(1, 2).reshape(-1, sh.hidden)
    h1 = X + F.linear(o_in, W[3])
    xm = F.rms_norm(h1, (sh.hidden,), eps=sh.eps)
    down_in = F.silu(F.linear(xm, W[4])) * F.linear(xm, W[5])
    out = h1 + F.linear(down_in, W[6])
    return [a.numpy() for a in (xa, o_in, xm, down_in)], out.numpy()


def test_rmsnorm_matches_library():
    x = np.random.default_rng(1).standard_normal((7, 33)) * 3
    for eps in (0.0, 1e-6, 0.5):
        want = F.rms_norm(torch.from_numpy(x), (33,), eps=eps).numpy()
        np.testing.assert_allclose(blk.rmsnorm(x, eps), want, rtol=1e-13, atol=0)
    y = blk.rmsnorm(x, 0.0)
    np.testing.assert_allclose(np.mean(y * y, axis=1), 1.0, rtol=1e-13)


def test_attention_matches_library():
    rng = np.random.default_rng(2)
    seqs, L, heads, dh = 3, 17, 4, 8
    q, k, v = (rng.standard_normal((seqs * L, heads * dh)) * 2 for _ in range(3))
    got = blk.causal_attention(q, k, v, seqs, L, heads)

    def hd(a):
        return torch.from_numpy(a).reshape(seqs, L, heads, dh).transpose(1, 2)

    want = F.scaled_dot_product_attention(hd(q), hd(k), hd(v), is_causal=True).transpose(1, 2).reshape(-1, heads * dh)
    np.testing.assert_allclose(got, want.numpy(), rtol=1e-12, atol=1e-13)
    # the first token of each sequence sees only itself
    np.testing.assert_allclose(got[::L], v[::L], rtol=1e-14)


def test_attention_uniform_weights_give_running_mean():
    rng = np.random.default_rng(3)
    seqs, L, heads, dh = 2, 9, 2, 4
    v = rng.standard_normal((seqs * L, heads * dh))
    zero = np.zeros_like(v)
    got = blk.causal_attention(zero, zero, v, seqs, L, heads)
    for s in range(seqs):
        vs = v[s * L:(s + 1) * L]
        want = np.cumsum(vs, axis=0) / np.arange(1, L + 1)[:, None]
        np.testing.assert_allclose(got[s * L:(s + 1) * L], want, rtol=1e-13, atol=1e-15)


def test_silu_matches_library():
    x = np.linspace(-30, 30, 301)
    np.testing.assert_allclose(blk.silu(x), F.silu(torch.from_numpy(x)).numpy(), rtol=1e-14, atol=1e-300)


def test_forward_matches_library_and_identity():
    rng = np.random.default_rng(4)
    X, W = _x(rng, SH), _weights(rng, SH)
    f = blk.forward(X, W, SH)
    li, lo = lib_forward(X, W, SH)
    for a, b in zip(f["inputs"], li):
        np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(f["out"], lo, rtol=1e-11, atol=1e-12)
    W0 = list(W)
    W0[3] = np.zeros_like(W[3])
    W0[6] = np.zeros_like(W[6])
    np.testing.assert_array_equal(blk.forward(X, W0, SH)["out"], X)


def _driver_checks(m, X, W, sh):
    """Names of the driver properties module m's quantize_block fails."""
    failed = []
    kw = dict(bits=2, group_size=16, block_size=8, act_order=True, damp=0.01)
    ts = m.quantize_block(X, W, sh, true_sequential=True, **kw)
    nts = m.quantize_block(X, W, sh, true_sequential=False, **kw)
    Qts = [lr.quant.Q for lr in ts.layers]
    Qnts = [lr.quant.Q for lr in nts.layers]
    # stage inputs, from the library forward through the weights each mode prescribes
    for si, members in enumerate(blk.STAGES):
        src = [Qts[i] if s < members[0] else W[i] for i, s in enumerate(range(7))]
        A_ts = lib_forward(X, src, sh)[0][si]
        A_nts = lib_forward(X, W, sh)[0][si]
        for mode, res, A in (("ts", ts, A_ts), ("nts", nts, A_nts)):
            H = 2.0 * A.T @ A
            if not np.allclose(res.hessians[si], H, rtol=1e-10, atol=1e-10 * np.abs(H).max()):
                failed.append(f"{mode} stage {si} input")
            for i in members:
                want = ref.gptq(W[i], None, 2, 16, 8, act_order=True, damp=0.01, H=H, n=A.shape[0])
                if not np.array_equal(res.layers[i].quant.codes, want.quant.codes):
                    failed.append(f"{mode} layer {blk.LAYERS[i]}")
    for i in (0, 1, 2):
        if not np.array_equal(ts.layers[i].quant.codes, nts.layers[i].quant.codes):
            failed.append("stage 0 depends on the mode")
    for mode, res, Q in (("ts", ts, Qts), ("nts", nts, Qnts)):
        if not np.allclose(res.out, lib_forward(X, Q, sh)[1], rtol=1e-10, atol=1e-10):
            failed.append(f"{mode} output")
    if all(np.array_equal(ts.layers[i].quant.codes, nts.layers[i].quant.codes) for i in range(3, 7)):
        failed.append("modes agree past stage 0")
    return failed


def test_driver_follows_the_stage_order():
    rng = np.random.default_rng(5)
    X, W = _x(rng, SH), _weights(rng, SH)
    assert _driver_checks(blk, X, W, SH) == []


MUTATIONS = [
    ("mask lets the next token in", "mask = np.triu(np.ones((seq_len, seq_len), dtype=bool), 1)",
     "mask = np.triu(np.ones((seq_len, seq_len), dtype=bool), 2)"),
    ("unscaled scores", "S = q[r, c] @ k[r, c].T / np.sqrt(dh)", "S = q[r, c] @ k[r, c].T"),
    ("attention residual dropped", "h1 = X + o_in @ W[3].T", "h1 = o_in @ W[3].T"),
    ("norm by the sum of squares", "np.mean(x * x, axis=1, keepdims=True)", "np.sum(x * x, axis=1, keepdims=True)"),
    ("silu sign", "return x / (1.0 + np.exp(-x))", "return x / (1.0 + np.exp(x))"),
    ("gate and up swapped", "down_in = silu(xm @ W[4].T) * (xm @ W[5].T)",
     "down_in = silu(xm @ W[5].T) * (xm @ W[4].T)"),
    ("quantized layers not fed forward", "cur[i] = layers[i].quant.Q", "pass"),
    ("output through the original weights", "out=forward(X, Wq, sh)[\"out\"]", "out=forward(X, W, sh)[\"out\"]"),
    ("o and gate/up stage inputs swapped", "A = forward(X, cur, sh)[\"inputs\"][si] if true_sequential",
     "A = forward(X, cur, sh)[\"inputs\"][3 - si if si in (1, 2) else si] if true_sequential"),
]


def _mutant(old, new):
    src = inspect.getsource(blk)
    assert src.count(old) >= 1, old
    src = src.replace("from . import gptq_ref as ref", "from oracle import gptq_ref as ref")
    mod = types.ModuleType("block_ref_mutant")
    sys.modules["block_ref_mutant"] = mod
    try:
        exec(compile(src.replace(old, new), "block_ref_mutant", "exec"), mod.__dict__)
    finally:
        sys.modules.pop("block_ref_mutant", None)
    return mod


def _piece_checks(m):
    failed = []
    rng = np.random.default_rng(6)
    X, W = _x(rng, SH), _weights(rng, SH)
    li, lo = lib_forward(X, W, SH)
    f = m.forward(X, W, SH)
    if not all(np.allclose(a, b, rtol=1e-10, atol=1e-12) for a, b in zip(f["inputs"], li)):
        failed.append("forward inputs")
    if not np.allclose(f["out"], lo, rtol=1e-10, atol=1e-12):
        failed.append("forward output")
    return failed


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, old, new):
    m = _mutant(old, new)
    failed = _piece_checks(m)
    if not failed:
        rng = np.random.default_rng(5)
        failed = _driver_checks(m, _x(rng, SH), _weights(rng, SH), SH)
    assert failed, f"planted mistake '{name}' passed every check"
