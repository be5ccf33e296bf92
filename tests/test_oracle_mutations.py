"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case edits one line of the oracle's source in memory (a dropped term, a wrong sign, a wrong
index, a transposed operand), loads the edited copy as a separate module and checks that at least
one pin-style check rejects it. The committed oracle is never modified.
"""

import inspect
import json
import os
import sys
import types
from fractions import Fraction

import numpy as np
import pytest

from oracle import gptq_ref as ref

HAND = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")))


def _f16_value(bits: int) -> float:
    """Value of an IEEE 754 binary16 bit pattern (5 exponent bits biased by 15, 10 fraction bits)."""
    e, m = (bits >> 10) & 0x1F, bits & 0x3FF
    v = m * 2.0 ** -24 if e == 0 else (1.0 + m / 1024.0) * 2.0 ** (e - 15)
    return -v if bits >> 15 else v

MUTATIONS = [
    ("drop lazy update", "Wp[:, e_blk:] -= Err @ Ub[:, e_blk:]", "pass"),
    ("wrong update sign", "Wp[:, i + 1:e_blk] -= np.outer(err, Ub[i - b, i + 1:e_blk])",
     "Wp[:, i + 1:e_blk] += np.outer(err, Ub[i - b, i + 1:e_blk])"),
    ("transposed factor row", "Wp[:, i + 1:e_blk] -= np.outer(err, Ub[i - b, i + 1:e_blk])",
     "Wp[:, i + 1:e_blk] -= np.outer(err, U[i + 1:e_blk, i])"),
    ("unscaled error", "err = (w - dq) / Ub[i - b, i]", "err = (w - dq)"),
    ("transposed lazy operand", "Wp[:, e_blk:] -= Err @ Ub[:, e_blk:]",
     "Wp[:, e_blk:] -= Err @ U[e_blk:, b:e_blk].T[:, :U.shape[0] - e_blk]"),
    ("factor block taken by columns", "Ub = np.asarray(U[b:e_blk], dtype=np.float64)",
     "Ub = np.asarray(U[:, b:e_blk].T, dtype=np.float64)"),
    ("grid from original weights", "s, z = grid_of(Wp[:, i:min(i + g, d)], gi)",
     "s, z = grid_of(W[:, perm][:, i:min(i + g, d)], gi)"),
    ("zero not added", "q = np.clip(_round_ratio(w, scale) + zero, 0.0, float(maxq))",
     "q = np.clip(_round_ratio(w, scale), 0.0, float(maxq))"),
    ("inverse not factored", "    u, info = lapack.dpotrf(inv, lower=0, clean=1)",
     "    u, info = np.triu(inv), 0"),
    ("damping on trace", "lam = float(damp) * mean_diag", "lam = float(damp) * mean_diag * d"),
    ("act-order ascending", "return np.argsort(-diag, kind=\"stable\").astype(np.int64)",
     "return np.argsort(diag, kind=\"stable\").astype(np.int64)"),
    ("hessian without factor 2", "H += 2.0 * (x.T @ x)", "H += (x.T @ x)"),
    ("pack nibble order", "words |= c[:, t::per].astype(np.uint64) << np.uint64(f * t)",
     "words |= c[:, t::per].astype(np.uint64) << np.uint64(f * (per - 1 - t))"),
    ("dense pack drops the straddling bits", "            words[:, w + 1] |= v >> np.uint64(32)",
     "            pass"),
    ("dense pack big-endian codes", "        v = c[:, k].astype(np.uint64) << np.uint64(sh)",
     "        v = c[:, d - 1 - k].astype(np.uint64) << np.uint64(sh)"),
    ("dequant zero not subtracted", "return s * (codes - z)", "return s * codes"),
    ("symmetric zero at code 0", "return scale, np.full(scale.shape, float((maxq + 1) // 2))",
     "return scale, np.zeros(scale.shape)"),
    ("symmetric scale from one side", "m = np.maximum(np.abs(wmin), np.abs(wmax))", "m = np.abs(wmax)"),
    ("static grid in processing order", "scales[:, gi], zeros[:, gi] = grid_of(W[:, cols], gi)",
     "scales[:, gi], zeros[:, gi] = grid_of(W[:, perm][:, cols], gi)"),
    ("compact scale not rounded to 16 bits", "    s = np.asarray(scale32, dtype=np.float32).astype(np.float16).astype(np.float64)",
     "    s = np.asarray(scale32, dtype=np.float64)"),
    ("compact zero not clamped", "        return scale, np.clip(_round_ratio(-wmin, scale), 0.0, float(maxq))",
     "        return scale, _round_ratio(-wmin, scale)"),
    ("static g_idx follows the order", "g_idx[:] = (np.arange(d) // g).astype(np.int32)",
     "g_idx[perm] = (np.arange(d) // g).astype(np.int32)"),
    ("dequant groups by position", "g = np.asarray(g_idx, dtype=np.int64)",
     "g = np.arange(d) * len(np.unique(g_idx)) // d"),
    ("dequant product transposed", "return np.asarray(x, dtype=np.float64) @ W.T",
     "return (np.asarray(x, dtype=np.float64)[:, :W.shape[0]] @ W).T"),
    ("brute force zero sign", "dq = s[r] * (grids - z[r])", "dq = s[r] * (grids + z[r])"),
    ("brute force drops the top code", "np.arange(maxq + 1, dtype=np.float64)", "np.arange(maxq, dtype=np.float64)"),
    ("brute force keeps the last row's optimum", "best += float(f[k])", "best = float(f[k])"),
    ("fp16 scale truncated", "    s = np.asarray(scale32, dtype=np.float32).astype(np.float16).astype(np.float64)",
     "    s = (np.asarray(scale32, dtype=np.float32).view(np.uint32) & np.uint32(0xFFFFE000)).view(np.float32)"
     ".astype(np.float16).astype(np.float64)"),
    ("follow scale window too wide", "def _follow_scale(own: np.ndarray, s32: np.ndarray, other: Optional[np.ndarray], rtol: float = 1e-5):",
     "def _follow_scale(own: np.ndarray, s32: np.ndarray, other: Optional[np.ndarray], rtol: float = 1e-2):"),
    ("follow scale takes any scale", "    return np.where(ok, other, own), int(np.count_nonzero(ok & (other != own)))",
     "    return other, int(np.count_nonzero(ok & (other != own)))"),
]


def _mutant(old, new):
    src = inspect.getsource(ref)
    assert src.count(old) >= 1, old
    mod = types.ModuleType("gptq_ref_mutant")
    sys.modules["gptq_ref_mutant"] = mod      # dataclasses look their module up by name
    try:
        exec(compile(src.replace(old, new), "gptq_ref_mutant", "exec"), mod.__dict__)
    finally:
        sys.modules.pop("gptq_ref_mutant", None)
    return mod


def _checks(m):
    """Return the names of the pin-style checks the module fails."""
    failed = []
    rng = np.random.default_rng(5)
    d, rows, n = 64, 8, 96
    z = rng.standard_normal((n, d))
    X = z @ (0.2 * np.eye(d) + 0.8 * rng.standard_normal((d, d)) / np.sqrt(d))
    X = X * rng.uniform(0.5, 2.0, d)[None, :]
    W = rng.standard_normal((rows, d)) * 0.02
    try:
        r = m.gptq(W, [X], 4, 16, 32, act_order=True, damp=0.01)
        p = r.quant.perm
        obj = ref.objective(W[:, p], r.quant.Q[:, p], r.Hhat)
        if not np.isclose(r.quant.loss, obj, rtol=1e-9):
            failed.append("loss identity")
        D = W - r.quant.Q
        if not np.isclose(np.sum((X @ D.T) ** 2), n / 2 * (r.quant.loss - r.lam * np.sum(D * D)), rtol=1e-8):
            failed.append("output identity")
        r1 = m.gptq(W, [X], 4, 16, 1, act_order=True, damp=0.01)
        if not np.array_equal(r1.quant.codes, r.quant.codes):
            failed.append("blocked == unblocked")
        if not np.allclose(r.U.T @ r.U @ r.Hhat, np.eye(d), atol=1e-8) or np.any(np.tril(r.U, -1) != 0):
            failed.append("factor")
        # each group's grid is the min/max grid of its weights as they stood at the group's first
        # column: original weights minus the closed-form total update Err[:, :k] @ U[:k, group]
        Wp = W[:, p]
        err = (r.quant.w_seen - r.quant.Q[:, p]) / np.diag(r.U)[None, :]
        for gi in range(1, d // 16):
            k = gi * 16
            cur = Wp[:, k:k + 16] - err[:, :k] @ r.U[:k, k:k + 16]
            s_want = np.maximum(cur.max(1) - cur.min(1), 1e-8) / 15
            if not np.allclose(r.quant.scales[:, gi], s_want, rtol=1e-9):
                failed.append("grid at group start")
                break
        if not np.all(np.diff(np.diag(r.H)[p]) <= 0):
            failed.append("act-order")
        Xi = rng.integers(-3, 4, size=(5, 4)).astype(np.float64)
        want = np.zeros((4, 4))
        for t in range(5):
            want += 2 * np.outer(Xi[t], Xi[t])
        if not np.array_equal(m.hessian([Xi])[0], want):
            failed.append("hessian definition")
        if m.pack(np.array([[1, 2, 3, 4, 5, 6, 7, 8]], np.uint8), 4)[0, 0] != np.array(
                [0x87654321], np.uint32).view(np.int32)[0]:
            failed.append("pack closed form")
        # a row's dense stream read as one integer is its codes as digits in base 2^bits
        cd = np.array([[k % 8 for k in range(32)]], np.uint8)
        pd = m.pack_dense(cd, 3).view(np.uint32).astype(object)
        if int(pd[0, 0] + (pd[0, 1] << 32) + (pd[0, 2] << 64)) != sum(int(cd[0, k]) << (3 * k) for k in range(32)):
            failed.append("dense pack positional value")
        Hs = np.diag([2.0, 4.0, 6.0]) * 10
        if not np.isclose(m.damp_and_order(Hs, 10, 0.01, False)[2], 0.04):
            failed.append("damping mean diag")
        q, _ = m.quantize_to_grid(np.array([0.75]), np.array([0.1]), np.array([2.0]), 15)
        if q[0] != 10:
            failed.append("grid primitive")
        # the stored layer, expanded and multiplied, worked by hand (interleaved groups)
        codes = np.array([list(range(16)), list(range(15, -1, -1))], np.uint8)
        xs = np.zeros((2, 16))
        xs[0, 0] = xs[0, 15] = 1.0
        xs[1, [0, 1, 2, 5, 12]] = [1.0, -1.0, 2.0, 0.5, -2.0]
        y = m.dequant_matmul(xs, ref.pack(codes, 4), np.array([[0.5, 0.25], [2.0, 1.0]]),
                             np.array([[2, 12], [8, 0]]), np.array([0, 0, 1, 1] * 4), 16)
        if y.shape != (2, 2) or not np.array_equal(y, np.array([[-0.25, 14.0], [-14.75, 50.0]])):
            failed.append("dequant hand example")
        # symmetric grids: H = I reduces to symmetric round-to-nearest; the zero is the middle code
        rs = m.gptq(W, None, 4, 16, 32, H=np.eye(d) * 2.0, n=1, sym=True)
        if not np.array_equal(rs.quant.codes, ref.rtn(W, 4, 16, sym=True).codes) or np.any(rs.quant.zeros != 8):
            failed.append("symmetric identity -> rtn")
        # static groups with act-order: H diagonal reduces to round-to-nearest over original columns
        Hd = np.diag(np.linspace(3.0, 1.0, d)[::-1]) * 2.0
        rst = m.gptq(W, None, 4, 16, 32, H=Hd, n=1, act_order=True, static_groups=True)
        if (not np.array_equal(rst.quant.codes, ref.rtn(W, 4, 16).codes)
                or not np.array_equal(rst.quant.g_idx, np.arange(d) // 16)):
            failed.append("static identity -> original-order rtn")
        # compact metadata: every scale is a float16 value, zeros fit the code width, and the
        # stored layer dequantizes to the weights the loop used
        Wc = W.copy()
        Wc[0] = np.abs(Wc[0]) + 0.05           # a one-signed row: its zero would lie below 0
        rc = m.gptq(Wc, [X], 4, 16, 32, act_order=True, damp=0.01, compact=True)
        qc = rc.quant
        if (not np.array_equal(qc.scales, qc.scales.astype(np.float16).astype(np.float64))
                or qc.zeros.min() < 0 or qc.zeros.max() > 15
                or not np.array_equal(ref.dequantize(ref.pack(qc.codes, 4), qc.scales, qc.zeros, qc.g_idx, d), qc.Q)):
            failed.append("compact metadata")
        # brute force: the hand-worked two-weight optimum (not round-to-nearest), and with a
        # diagonal Hessian the separable minimum, round-to-nearest's weighted error
        e = HAND["brute_force_two_weights"]
        Wb = np.array([[float(Fraction(v)) for v in e["weights"]]])
        Hb = np.array([[float(Fraction(v)) for v in r] for r in e["hhat"]])
        fb, Qb = m.brute_force(Wb, Hb, 2)
        if (not np.isclose(fb, float(Fraction(e["optimal_objective"])), rtol=1e-12)
                or not np.allclose(Qb[0], [float(Fraction(v)) for v in e["optimal_values"]], atol=1e-15)):
            failed.append("brute force hand example")
        Wd = W[:3, :5] + 0.01
        hd = np.linspace(0.5, 4.0, 5)
        fd, _ = m.brute_force(Wd, np.diag(hd), 2)
        if not np.isclose(fd, np.sum(hd[None, :] * (Wd - ref.rtn(Wd, 2, 0).Q) ** 2), rtol=1e-12):
            failed.append("brute force diagonal -> rtn")
        # 16-bit scales: hand-derived float16 patterns, and the boundary rule of following
        for c in HAND["float16_scale_rounding"]["cases"]:
            x = float(Fraction(c["exact"]))
            with np.errstate(over="ignore"):
                got = m.fp16_scale(np.array([x]))[0]
            if got != _f16_value(int(c["float16"], 16)):
                failed.append("fp16 scale bit patterns")
                break
        mid = float(Fraction(2049, 2048))
        own = m.fp16_scale(np.array([mid]))
        far = 1.0 + 2.0 ** -12
        if (m._follow_scale(own, np.array([mid]), np.array([_f16_value(0x3C02)]))[0][0] != own[0]
                or m._follow_scale(m.fp16_scale(np.array([far])), np.array([far]),
                                   np.array([_f16_value(0x3C01)]))[0][0] != 1.0
                or m._follow_scale(own, np.array([mid]), np.array([_f16_value(0x3C01)]))[0][0] != _f16_value(0x3C01)):
            failed.append("follow scale boundary")
        # H = I must reduce to round-to-nearest with dynamic grids
        rI = m.gptq(W, None, 4, 16, 32, H=np.eye(d) * 2.0, n=1)
        if not np.array_equal(rI.quant.codes, ref.rtn(W, 4, 16).codes):
            failed.append("identity -> rtn")
    except Exception as e:  # a crash is also a rejection
        failed.append(f"raised {type(e).__name__}")
    return failed


def test_unmodified_oracle_passes_checks():
    assert _checks(ref) == []


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, old, new):
    assert _checks(_mutant(old, new)), name
