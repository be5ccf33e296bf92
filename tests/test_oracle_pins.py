"""Pins of the float64 oracle against what the pages and the mathematics fix (CPU only).

Each test names the passage or the closed form it checks. Together they are chosen so that a
dropped term, a wrong sign or index, or a transposed operand anywhere in the oracle fails one of them.
"""

import itertools
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import gptq_ref as ref

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))
HAND = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")))


def _correlated_x(rng, n, d, mix=0.8):
    z = rng.standard_normal((n, d))
    m = np.eye(d) * (1 - mix) + mix * rng.standard_normal((d, d)) / np.sqrt(d)
    return z @ m


def _solve(W, X, bits, g, B, act=False, damp=0.01):
    return ref.gptq(W, [X], bits, g, B, act_order=act, damp=damp)


# ---------------------------------------------------------------- grid primitive (page examples)

def test_quantization_equation_example():
    e = GOLD["quantization_equation"]
    q, dq = ref.quantize_to_grid(np.array([e["original"]]), np.array([e["scale"]]), np.array([0.0]), 15)
    assert q[0] == e["quantized"]
    assert dq[0] == pytest.approx(e["recovered"], abs=1e-15)
    assert abs(e["original"] - dq[0]) == pytest.approx(e["abs_error"], abs=1e-15)


def test_quantization_equation_through_solver():
    # A row whose min/max are 0 and 1.5 at 4 bits has scale 1.5/15 = 0.1; with H = I there is no
    # feedback, so the weight 0.75 must take code 8 (value 0.8).
    W = np.array([[0.0, 1.5, 0.75, 0.3]])
    X = np.eye(4) * np.sqrt(0.5)          # 2 X^T X = I
    r = ref.gptq(W, [X], 4, 0, 4, damp=0.01, H=np.eye(4) * 4.0, n=4)
    assert r.quant.scales[0, 0] == pytest.approx(0.1, rel=1e-15)
    assert r.quant.zeros[0, 0] == 0
    assert r.quant.codes[0, 2] == 8
    assert r.quant.Q[0, 2] == pytest.approx(0.8, abs=1e-15)


def test_single_weight_example():
    e = GOLD["single_weight"]
    q, dq = ref.quantize_to_grid(np.array([e["original"]]), np.array([e["scale"]]), np.array([0.0]), 15)
    assert q[0] == e["quantized"]
    assert dq[0] == pytest.approx(e["dequantized"], abs=1e-15)
    assert e["original"] - dq[0] == pytest.approx(e["error"], abs=1e-12)


def test_two_weight_correlated_example():
    e = GOLD["two_weights"]
    rho = e["correlation_near_one"]
    Hh = np.array([[1.0, rho], [rho, 1.0]])
    U = ref.inverse_cholesky_upper(Hh)
    W = np.array([e["weights"]])
    step = e["grid_step"]
    grid = (np.full((1, 1), step), np.zeros((1, 1)))
    r = ref.quantize_layer(W, U, 2, 0, 2, grid=grid)
    # first weight rounds as RTN does
    assert r.Q[0, 0] == pytest.approx(e["rtn"][0], abs=1e-15)
    # the correction reduces the second weight: 0.31 - 0.1 * rho = 0.2101, "about 0.21"
    w2 = r.w_seen[0, 1]
    assert w2 == pytest.approx(0.31 - 0.1 * rho, abs=1e-12)
    assert abs(w2 - e["second_weight_after_correction_about"]) < 0.005
    assert r.Q[0, 1] == pytest.approx(e["second_weight_rounds_to"], abs=1e-15)
    # plain rounding of the pair and its errors
    rq = np.rint(W / step) * step
    assert np.allclose(rq[0], e["rtn"], atol=1e-15)
    assert np.allclose(rq[0] - W[0], e["rtn_errors"], atol=1e-12)


# ---------------------------------------------------------------- reductions to RTN

@pytest.mark.parametrize("g,B", [(16, 32), (32, 16), (0, 16), (64, 64)])
def test_identity_hessian_is_rtn(g, B):
    rng = np.random.default_rng(11)
    W = rng.standard_normal((24, 64)) * 0.02
    r = ref.gptq(W, None, 4, g, B, H=np.eye(64) * 2.0, n=1)
    t = ref.rtn(W, 4, g)
    assert np.array_equal(r.quant.codes, t.codes)
    assert np.allclose(r.quant.scales, t.scales, rtol=0, atol=0)
    assert np.array_equal(r.quant.zeros, t.zeros)


@pytest.mark.parametrize("act", [False, True])
def test_diagonal_hessian_is_rtn(act):
    rng = np.random.default_rng(12)
    d = 48
    W = rng.standard_normal((10, d)) * 0.02
    H = np.diag(rng.uniform(0.5, 4.0, d))
    r = ref.gptq(W, None, 3, 16, 16, act_order=act, H=H, n=1)
    t = ref.rtn(W, 3, 16, perm=r.quant.perm)
    assert np.array_equal(r.quant.codes, t.codes)
    if act:
        assert not np.array_equal(r.quant.perm, np.arange(d))


# ---------------------------------------------------------------- loss identities

@pytest.mark.parametrize("bits,g,B,act", [(4, 16, 32, False), (3, 0, 16, False), (2, 8, 8, True), (4, 32, 16, True)])
def test_loss_identity(bits, g, B, act):
    """sum err^2 == sum_r (W-Q)_r Hhat (W-Q)_r^T, and == (2/n)||X (W-Q)^T||^2 + lam ||W-Q||^2.

    The sequential updates are exact minimisers of the damped quadratic over the not yet quantized
    columns (tools page, Steps 5-6), so the accumulated squared scaled errors equal the objective.
    """
    rng = np.random.default_rng(100 + bits + g + B)
    d, rows, n = 64, 12, 96
    X = _correlated_x(rng, n, d)
    W = rng.standard_normal((rows, d)) * 0.02
    r = _solve(W, X, bits, g, B, act)
    p = r.quant.perm
    obj = ref.objective(W[:, p], r.quant.Q[:, p], r.Hhat)
    assert r.quant.loss == pytest.approx(obj, rel=1e-10)
    D = W - r.quant.Q
    outputs = np.sum((X @ D.T) ** 2)
    assert outputs == pytest.approx(n / 2 * (r.quant.loss - r.lam * np.sum(D * D)), rel=1e-9)


def test_cholesky_rows_are_sequential_inverse():
    """U[k,k]^2 = [Hhat_FF^-1]_kk and U[k,F]/U[k,k] = Hhat_FF^-1[k,:]/[Hhat_FF^-1]_kk, F = {k..d-1}."""
    rng = np.random.default_rng(3)
    d = 12
    X = _correlated_x(rng, 40, d)
    Hh = 2 * X.T @ X / 40 + 0.01 * np.eye(d)
    U = ref.inverse_cholesky_upper(Hh)
    for k in range(d):
        inv = np.linalg.inv(Hh[k:, k:])
        assert U[k, k] ** 2 == pytest.approx(inv[0, 0], rel=1e-10)
        assert np.allclose(U[k, k:] / U[k, k], inv[0, :] / inv[0, 0], rtol=1e-9, atol=1e-12)


def test_factor_properties():
    rng = np.random.default_rng(4)
    d = 40
    X = _correlated_x(rng, 200, d)
    Hh = 2 * X.T @ X / 200 + 0.05 * np.eye(d)
    U = ref.inverse_cholesky_upper(Hh)
    assert np.allclose(np.tril(U, -1), 0)
    assert np.all(np.diag(U) > 0)
    assert np.allclose(U.T @ U @ Hh, np.eye(d), atol=1e-10)
    # the reversed-order route: U = J chol(J Hhat J)^-1 J
    J = np.eye(d)[::-1]
    U2 = J @ np.linalg.inv(np.linalg.cholesky(J @ Hh @ J)) @ J
    assert np.allclose(U, U2, rtol=1e-9, atol=1e-12)


# ---------------------------------------------------------------- lazy blocks

@pytest.mark.parametrize("act", [False, True])
def test_blocked_equals_unblocked(act):
    """Lazy batching is a reorganisation (tools page, Step 7): every nesting block size gives the
    same codes as the column-at-a-time loop."""
    rng = np.random.default_rng(21)
    d, rows = 128, 16
    X = _correlated_x(rng, 160, d)
    W = rng.standard_normal((rows, d)) * 0.02
    base = _solve(W, X, 4, 32, 1, act)
    for B in (8, 32, 64, 128):
        r = _solve(W, X, 4, 32, B, act)
        assert np.array_equal(r.quant.codes, base.quant.codes), B
        assert np.array_equal(r.quant.zeros, base.quant.zeros), B
        assert r.quant.loss == pytest.approx(base.quant.loss, rel=1e-10)


def test_ragged_block_and_group():
    rng = np.random.default_rng(22)
    d = 100   # last block and last group are short
    X = _correlated_x(rng, 150, d)
    W = rng.standard_normal((8, d)) * 0.02
    a = _solve(W, X, 4, 16, 32)
    b = _solve(W, X, 4, 16, 1)
    assert a.quant.scales.shape == (8, 7)
    assert np.array_equal(a.quant.codes, b.quant.codes)
    p = a.quant.perm
    assert a.quant.loss == pytest.approx(ref.objective(W[:, p], a.quant.Q[:, p], a.Hhat), rel=1e-10)


def test_group_grid_is_taken_from_updated_weights():
    """Each group's grid is the min/max grid of its weights as they stand at the group's first
    column (the reading taken for when a grid is computed). The weights at that moment are
    reconstructed independently: the original weights minus the closed-form total update
    Err[:, :k] @ U[:k, group] from every earlier column k, whatever the blocking."""
    rng = np.random.default_rng(23)
    d, g = 64, 8
    X = _correlated_x(rng, 80, d)
    W = rng.standard_normal((6, d)) * 0.02
    for B in (8, 32, 64):
        r = _solve(W, X, 4, g, B)
        err = (r.quant.w_seen - r.quant.Q) / np.diag(r.U)[None, :]
        for gi in range(d // g):
            k = gi * g
            cur = W[:, k:k + g] - err[:, :k] @ r.U[:k, k:k + g]
            s_want = np.maximum(cur.max(1) - cur.min(1), 1e-8) / 15
            z_want = np.rint((-cur.min(1)).astype(np.float32) / s_want.astype(np.float32))
            assert np.allclose(r.quant.scales[:, gi], s_want, rtol=1e-9)
            assert np.array_equal(r.quant.zeros[:, gi], z_want.astype(np.int32))
    t = ref.rtn(W, 4, g)
    assert np.allclose(r.quant.scales[:, 0], t.scales[:, 0], rtol=0, atol=0)
    assert not np.allclose(r.quant.scales[:, 1:], t.scales[:, 1:])


# ---------------------------------------------------------------- optimality checks

def test_no_lower_than_brute_force():
    """On layers of <= 8 weights at 2 bits the solver's objective is >= the exhaustive optimum over
    the same per-row grid (tools page, Step 2 objective)."""
    rng = np.random.default_rng(31)
    for trial in range(150):
        d = int(rng.integers(2, 9))
        X = _correlated_x(rng, 3 * d, d, mix=0.9)
        W = rng.standard_normal((2, d)) * 0.02
        r = _solve(W, X, 2, 0, d)
        best, _ = ref.brute_force(W, r.Hhat, 2)
        obj = ref.objective(W, r.quant.Q, r.Hhat)
        assert obj >= best * (1 - 1e-12) - 1e-18, trial
        assert obj == pytest.approx(r.quant.loss, rel=1e-9)


def test_brute_force_hand_worked_instance():
    """The exhaustive optimum of a two-weight 2-bit row worked by hand (tests/golden/hand_worked.json):
    the 16 code pairs enumerated here in exact rational arithmetic, then found by brute_force. Its
    optimum is not round-to-nearest, so a search that returned round-to-nearest would fail."""
    e = HAND["brute_force_two_weights"]
    w = [Fraction(v) for v in e["weights"]]
    Hh = [[Fraction(v) for v in r] for r in e["hhat"]]
    maxq = (1 << e["bits"]) - 1
    s, z = Fraction(e["scale"]), e["zero"]
    assert s == (max(w) - min(w)) / maxq                       # the row's min/max grid
    assert abs(-min(w) / s - z) <= Fraction(1, 2)                # the zero is the nearest integer

    def f(q):
        D = [w[i] - s * (q[i] - z) for i in range(2)]
        return sum(D[i] * Hh[i][j] * D[j] for i in range(2) for j in range(2))

    table = sorted((f(q), q) for q in itertools.product(range(maxq + 1), repeat=2))
    assert table[0] == (Fraction(e["optimal_objective"]), tuple(e["optimal_codes"]))
    assert table[1][0] > table[0][0]                            # a unique optimum
    assert f(tuple(e["rtn_codes"])) == Fraction(e["rtn_objective"])
    W = np.array([[float(v) for v in w]])
    H64 = np.array([[float(v) for v in r] for r in Hh])
    best, Q = ref.brute_force(W, H64, e["bits"])
    assert best == pytest.approx(float(Fraction(e["optimal_objective"])), rel=1e-12)
    assert np.allclose(Q[0], [float(Fraction(v)) for v in e["optimal_values"]], rtol=0, atol=1e-15)
    t = ref.rtn(W, e["bits"], 0)
    assert list(t.codes[0]) == e["rtn_codes"]


@pytest.mark.parametrize("bits", [2, 3])
def test_brute_force_with_diagonal_hessian_is_rtn(bits):
    """With a diagonal Hhat the objective is sum_j h_j (w_j - q_j)^2, each term minimised on its own
    by the grid value nearest w_j, so the exhaustive optimum is round-to-nearest's error, written out
    here as that sum."""
    rng = np.random.default_rng(38 + bits)
    for trial in range(120):
        d = int(rng.integers(2, 7 if bits == 2 else 6))
        W = rng.standard_normal((3, d)) * 0.02 + rng.uniform(-0.02, 0.02, (3, 1))
        h = rng.uniform(0.1, 10.0, d)
        best, Q = ref.brute_force(W, np.diag(h), bits)
        t = ref.rtn(W, bits, 0)
        want = float(np.sum(h[None, :] * (W - t.Q) ** 2))
        assert best == pytest.approx(want, rel=1e-12, abs=1e-30), trial
        assert np.allclose(Q, t.Q, rtol=0, atol=1e-15), trial


def _f16_value(bits: int) -> float:
    """Value of an IEEE 754 binary16 bit pattern: sign bit, 5 exponent bits biased by 15, 10 fraction
    bits; exponent field 0 holds the subnormals m 2^-24."""
    e, m = (bits >> 10) & 0x1F, bits & 0x3FF
    assert e != 0x1F
    v = m * 2.0 ** -24 if e == 0 else (1.0 + m / 1024.0) * 2.0 ** (e - 15)
    return -v if bits >> 15 else v


@pytest.mark.filterwarnings("ignore:overflow encountered in cast")
def test_fp16_scale_hand_derived_bit_patterns():
    """Compact scales round to the nearest float16, ties to even, with zero and overflow kept inside
    the finite positive range: each case's float16 bit pattern is derived by hand in
    tests/golden/hand_worked.json (exact midpoints included)."""
    for c in HAND["float16_scale_rounding"]["cases"]:
        x = float(Fraction(c["exact"]))
        assert float(np.float32(x)) == x or c["exact"] in ("2/15", "1/150"), c["value"]
        got = ref.fp16_scale(np.array([x]))[0]
        assert got == _f16_value(int(c["float16"], 16)), c["value"]


def test_follow_scale_adopts_only_at_float16_boundaries():
    """_follow_scale may replace this oracle's 16-bit scale by the other side's only when the float32
    scale lies within rtol of a float16 rounding boundary and the other scale is one of the two
    float16 values around it."""
    one, nxt, nxt2 = _f16_value(0x3C00), _f16_value(0x3C01), _f16_value(0x3C02)
    mid = float(Fraction(2049, 2048))                 # the midpoint of 0x3C00 and 0x3C01
    own = ref.fp16_scale(np.array([mid]))
    assert own[0] == one                              # ties to even
    out, n = ref._follow_scale(own, np.array([mid]), np.array([nxt]))
    assert out[0] == nxt and n == 1                   # the other neighbour: adopted and counted
    out, n = ref._follow_scale(own, np.array([mid]), np.array([one]))
    assert out[0] == one and n == 0                   # the same choice: nothing counted
    out, n = ref._follow_scale(own, np.array([mid]), np.array([nxt2]))
    assert out[0] == one and n == 0                   # not a neighbour: refused
    near = mid * (1.0 + 2.0 ** -21)                   # 4.8e-7 above the boundary: inside rtol
    own_n = ref.fp16_scale(np.array([near]))
    assert own_n[0] == nxt
    out, n = ref._follow_scale(own_n, np.array([near]), np.array([one]))
    assert out[0] == one and n == 1
    far = 1.0 + 2.0 ** -12                            # 2.4e-4 from the nearest boundary: outside rtol
    own_f = ref.fp16_scale(np.array([far]))
    out, n = ref._follow_scale(own_f, np.array([far]), np.array([nxt]))
    assert out[0] == own_f[0] == one and n == 0       # refused although a neighbour
    out, n = ref._follow_scale(own, np.array([mid]), None)
    assert out[0] == one and n == 0


def test_two_weight_never_worse_than_rtn():
    """d = 2, one group: the second code is the nearest grid point to the conditional optimum, so the
    damped objective can only improve on round-to-nearest."""
    rng = np.random.default_rng(32)
    for _ in range(1000):
        X = _correlated_x(rng, 4, 2, mix=0.95)
        W = rng.standard_normal((1, 2)) * 0.02
        r = _solve(W, X, 2, 0, 2)
        t = ref.rtn(W, 2, 0)
        assert ref.objective(W, r.quant.Q, r.Hhat) <= ref.objective(W, t.Q, r.Hhat) * (1 + 1e-12) + 1e-20


@pytest.mark.parametrize("d", [4, 8])
def test_better_than_rtn_in_aggregate(d):
    """GPTQ beats round-to-nearest in aggregate over seeded correlated layers (Paper breakdown, The
    Problem; tools page remark after the sketch). Per instance it can lose, so only the sum is asserted."""
    rng = np.random.default_rng(33 + d)
    g_sum = r_sum = 0.0
    worse = 0
    for _ in range(1000):
        X = _correlated_x(rng, 2 * d, d, mix=0.9)
        W = rng.standard_normal((1, d)) * 0.02
        r = _solve(W, X, 2, 0, d)
        t = ref.rtn(W, 2, 0)
        a = ref.objective(W, r.quant.Q, r.Hhat)
        b = ref.objective(W, t.Q, r.Hhat)
        g_sum += a
        r_sum += b
        worse += a > b * (1 + 1e-12)
    assert g_sum < 0.9 * r_sum
    assert worse < 500


# ---------------------------------------------------------------- act-order

def test_act_order_descending_diag_is_identity_order():
    rng = np.random.default_rng(41)
    d = 32
    X = _correlated_x(rng, 100, d)
    X = X[:, np.argsort(-np.sum(X * X, axis=0))]       # features already in descending diag order
    W = rng.standard_normal((8, d)) * 0.02
    H, n = ref.hessian([X])
    assert np.all(np.diff(np.diag(H)) < 0)
    a = ref.gptq(W, None, 4, 8, 8, act_order=True, H=H, n=n)
    b = ref.gptq(W, None, 4, 8, 8, act_order=False, H=H, n=n)
    assert np.array_equal(a.quant.perm, np.arange(d))
    assert np.array_equal(a.quant.codes, b.quant.codes)


def test_act_order_permutation_equivariance():
    """Permuting input features (W columns and X columns together) leaves act-order results unchanged
    up to that permutation when diag(H) has no ties."""
    rng = np.random.default_rng(42)
    d = 48
    X = _correlated_x(rng, 120, d)
    W = rng.standard_normal((8, d)) * 0.02
    sig = rng.permutation(d)
    a = _solve(W, X, 4, 16, 16, act=True)
    b = _solve(W[:, sig], X[:, sig], 4, 16, 16, act=True)
    assert np.array_equal(b.quant.codes, a.quant.codes[:, sig])
    assert np.array_equal(b.quant.g_idx, a.quant.g_idx[sig])
    assert np.array_equal(sig[b.quant.perm], a.quant.perm)
    assert b.quant.loss == pytest.approx(a.quant.loss, rel=1e-12)


def test_act_order_ties_keep_lower_index_first():
    H = np.diag([1.0, 3.0, 1.0, 3.0, 2.0])
    assert list(ref.act_order_perm(H)) == [1, 3, 4, 0, 2]


def test_g_idx_maps_original_columns_to_processing_groups():
    rng = np.random.default_rng(43)
    d = 32
    X = _correlated_x(rng, 64, d) * rng.uniform(0.5, 2, d)[None, :]
    W = rng.standard_normal((4, d)) * 0.02
    r = _solve(W, X, 4, 8, 8, act=True)
    p = r.quant.perm
    for j in range(d):
        assert r.quant.g_idx[p[j]] == j // 8


# ---------------------------------------------------------------- Hessian

def test_hessian_matches_definition_exactly():
    """H = sum over tokens of 2 x x^T (Technical Guide, Computing the Hessian), small integers so the
    float64 sums are exact; chunked accumulation equals the one-shot sum."""
    rng = np.random.default_rng(51)
    X = rng.integers(-3, 4, size=(7, 5)).astype(np.float64)
    want = [[0.0] * 5 for _ in range(5)]
    for t in range(7):
        for i in range(5):
            for j in range(5):
                want[i][j] += 2.0 * X[t, i] * X[t, j]
    H, n = ref.hessian([X[:3], X[3:5], X[5:]])
    assert n == 7
    assert np.array_equal(H, np.array(want))
    H1, _ = ref.hessian([X])
    assert np.array_equal(H, H1)


def test_damping_is_mean_of_diagonal():
    H = np.diag([2.0, 4.0, 6.0]) * 10
    Hh, perm, lam = ref.damp_and_order(H, 10, 0.01, False)
    assert lam == pytest.approx(0.04, rel=1e-15)
    assert np.allclose(np.diag(Hh), [2.04, 4.04, 6.04], rtol=1e-15)


# ---------------------------------------------------------------- packing and format

def test_pack_closed_form():
    codes = np.array([[1, 2, 3, 4, 5, 6, 7, 8], [15] * 8, [0] * 8], dtype=np.uint8)
    p = ref.pack(codes, 4)
    assert p.dtype == np.int32
    assert p[0, 0] == np.array([0x87654321], dtype=np.uint32).view(np.int32)[0]
    assert p[1, 0] == -1
    assert p[2, 0] == 0
    for k in range(3):
        for t in range(8):
            c = np.zeros((1, 24), dtype=np.uint8)
            c[0, 8 * k + t] = 1
            w = ref.pack(c, 4)
            assert w[0, k] == np.int32(1 << (4 * t))
            assert np.count_nonzero(w) == 1


def test_pack_round_trip():
    rng = np.random.default_rng(61)
    for bits in (2, 3, 4):
        c = rng.integers(0, 1 << bits, size=(5, 64)).astype(np.uint8)
        assert np.array_equal(ref.unpack(ref.pack(c, bits), 64), c)
    with pytest.raises(ValueError):
        ref.pack(np.full((1, 8), 8, np.uint8), 3)


def test_format_overhead():
    e = GOLD["memory_arithmetic"]
    bpw = ref.bits_per_weight(e["bits"], e["group_size"], e["scale_bits"], e["zero_bits"])
    assert round(bpw, 2) == e["bits_per_weight_about"]
    assert round(bpw - e["bits"], 2) == e["overhead_bits_per_weight_about"]
    ratio = (ref.bits_per_weight(4, 32) - 4) / (bpw - 4)
    assert ratio == pytest.approx(e["group32_overhead_ratio_about"])
    assert GOLD["packing"]["codes_per_word"] * 4 == GOLD["packing"]["word_bits"]


# ---------------------------------------------------------------- failure paths and edge cases

def test_rank_deficient_undamped_fails_with_pivot():
    """A dead feature with no damping leaves the Hessian singular (tools page, "When the method
    breaks down"; "Forgetting damping"): the factor reports the failing pivot."""
    rng = np.random.default_rng(71)
    X = rng.standard_normal((50, 6))
    X[:, 3] = 0.0
    H, n = ref.hessian([X])
    Hh, _, _ = ref.damp_and_order(H, n, 0.0, False)
    with pytest.raises(ref.NotPositiveDefinite) as ei:
        ref.inverse_cholesky_upper(Hh)
    assert ei.value.pivot == 4
    # damping repairs it
    Hh, _, _ = ref.damp_and_order(H, n, 0.01, False)
    ref.inverse_cholesky_upper(Hh)


def test_rejected_shapes():
    with pytest.raises(ValueError):
        ref.check_geometry(64, 1, 16)          # group_size 1 (Technical Guide, Don'ts)
    with pytest.raises(ValueError):
        ref.check_geometry(64, 24, 16)         # groups and blocks do not nest
    with pytest.raises(ValueError):
        ref.damp_and_order(np.zeros((4, 4)), 1, 0.01, False)


def test_constant_group():
    W = np.full((2, 8), 0.3)
    W[1] = -0.7
    r = ref.gptq(W, None, 4, 0, 8, H=np.eye(8), n=1)
    assert np.allclose(r.quant.scales, 1e-8 / 15)
    assert np.all(r.quant.codes == 0)
    assert np.allclose(r.quant.Q, W, atol=1e-9)


def test_follow_adopts_only_inside_tie_window():
    """The follow mode used by parity tests may only change decisions that lie inside the tie window."""
    rng = np.random.default_rng(81)
    d = 64
    X = _correlated_x(rng, 100, d)
    W = rng.standard_normal((16, d)) * 0.02
    base = _solve(W, X, 4, 16, 16)
    flipped = base.quant.codes_proc.astype(np.int64)
    flipped = np.where(flipped < 15, flipped + 1, flipped - 1)    # every code moved by one
    r = ref.quantize_layer(W, base.U, 4, 16, 16, follow=(flipped, base.quant.zeros), tau=1e-3)
    # only near-tie decisions may be adopted; with a tiny window almost none are
    assert r.adopted_diff <= r.near_ties
    r0 = ref.quantize_layer(W, base.U, 4, 16, 16, follow=(flipped, base.quant.zeros), tau=0.0)
    assert r0.adopted == 0
    assert np.array_equal(r0.codes, base.quant.codes)
    rall = ref.quantize_layer(W, base.U, 4, 16, 16, follow=(flipped, base.quant.zeros), tau=0.5)
    assert rall.adopted_diff > 0


# ---------------------------------------------------------------- using the stored layer (Step 8)

def test_dequantize_worked_example_values():
    """Technical Guide, 'Quantization Equation' and 'Example: Quantizing a Single Weight': code 8 at
    scale 0.1 recovers 0.8, code 7 recovers 0.7 (zero point 0)."""
    e1, e2 = GOLD["quantization_equation"], GOLD["single_weight"]
    codes = np.zeros((1, 8), np.uint8)
    codes[0, 0], codes[0, 5] = e1["quantized"], e2["quantized"]
    w = ref.dequantize(ref.pack(codes, 4), np.array([[0.1]]), np.array([[0]]), np.zeros(8, np.int32), 8)
    assert w[0, 0] == pytest.approx(e1["recovered"], abs=1e-15)
    assert w[0, 5] == pytest.approx(e2["dequantized"], abs=1e-15)
    assert np.all(w[0, [1, 2, 3, 4, 6, 7]] == 0)


def test_dequant_matmul_hand_example():
    """y = x W^T with W[r, j] = s[r, g_idx[j]] (code - z[r, g_idx[j]]), worked by hand on two rows of
    16 columns whose groups interleave (as act-order leaves them)."""
    codes = np.array([list(range(16)), list(range(15, -1, -1))], np.uint8)
    g_idx = np.array([0, 0, 1, 1] * 4, np.int32)
    s = np.array([[0.5, 0.25], [2.0, 1.0]])
    z = np.array([[2, 12], [8, 0]], np.int32)
    x = np.zeros((2, 16))
    x[0, 0] = x[0, 15] = 1.0
    x[1, [0, 1, 2, 5, 12]] = [1.0, -1.0, 2.0, 0.5, -2.0]
    y = ref.dequant_matmul(x, ref.pack(codes, 4), s, z, g_idx, 16)
    # row 0 weights at columns 0, 1, 2, 5, 12, 15: .5(0-2), .5(1-2), .25(2-12), .5(5-2), .5(12-2), .25(15-12)
    # row 1 weights at the same columns: 2(15-8), 2(14-8), 1(13-0), 2(10-8), 2(3-8), 1(0-0)
    want = np.array([[-1.0 + 0.75, 14.0 + 0.0],
                     [1 * -1.0 - 1 * -0.5 + 2 * -2.5 + 0.5 * 1.5 - 2 * 5.0,
                      1 * 14.0 - 1 * 12.0 + 2 * 13.0 + 0.5 * 4.0 - 2 * -10.0]])
    assert np.array_equal(y, want)


@pytest.mark.parametrize("act", [False, True])
def test_dequantize_reproduces_column_loop_weights(act):
    """Unpacking the codes and expanding each column with its group's scale and zero gives exactly
    the weights the column loop dequantized, in the original column order, with or without act-order."""
    rng = np.random.default_rng(17)
    d = 64
    X = _correlated_x(rng, 96, d) * rng.uniform(0.3, 3.0, d)[None, :]
    W = rng.standard_normal((12, d)) * 0.02
    r = _solve(W, X, 4, 16, 32, act=act)
    q = r.quant
    w = ref.dequantize(ref.pack(q.codes, 4), q.scales, q.zeros, q.g_idx, d)
    assert np.array_equal(w, q.Q)
    y = ref.dequant_matmul(X[:5], ref.pack(q.codes, 4), q.scales, q.zeros, q.g_idx, d)
    assert np.allclose(y, X[:5] @ q.Q.T, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- symmetric grid and static groups

def test_symmetric_grid_single_weight_example():
    """Technical Guide, 'Example: Quantizing a Single Weight': int4 range [-8, 7], scale 0.1, the weight
    0.7382594 takes the signed code 7 and dequantizes to 0.7 (error 0.0382594). As unsigned codes with
    the symmetric zero 8 that is code 15."""
    e = GOLD["single_weight"]
    q, dq = ref.quantize_to_grid(np.array([e["original"]]), np.array([e["scale"]]), np.array([8.0]), 15)
    assert q[0] - 8 == e["quantized"]
    assert dq[0] == pytest.approx(e["dequantized"], abs=1e-12)
    assert e["original"] - dq[0] == pytest.approx(e["error"], abs=1e-12)
    _, z = ref.group_grid(np.array([[-0.2, 0.5]]), 15, sym=True)
    assert z[0] == 8                                   # the middle code of [0, 15], signed range [-8, 7]


@pytest.mark.parametrize("bits,zero", [(4, 8), (3, 4), (2, 2)])
def test_symmetric_grid_closed_form(bits, zero):
    maxq = (1 << bits) - 1
    wg = np.array([[-0.3, 0.7, 0.1], [-0.9, 0.2, 0.0], [0.0, 0.0, 0.0]])
    s, z = ref.group_grid(wg, maxq, sym=True)
    assert np.allclose(s, [1.4 / maxq, 1.8 / maxq, 1e-8 / maxq], rtol=1e-15)
    assert np.all(z == zero)
    # values are (code - zero) steps, so the range is [-zero, maxq - zero] steps: the positive
    # extreme m = 0.9 (m / s = maxq / 2) clips to maxq - zero steps; 0.2 rounds to nearest
    q, dq = ref.quantize_to_grid(np.array([0.9, 0.2]), s[[1, 1]], z[[1, 1]], maxq)
    assert q[0] == maxq and dq[0] == pytest.approx((maxq - zero) * 1.8 / maxq)
    assert q[1] == zero + np.rint(0.2 * maxq / 1.8) and dq[1] == pytest.approx((q[1] - zero) * 1.8 / maxq)


def test_symmetric_identity_hessian_is_rtn():
    """With H = I there is no error feedback: symmetric GPTQ equals symmetric round-to-nearest."""
    rng = np.random.default_rng(23)
    W = rng.standard_normal((8, 64)) * 0.02
    r = ref.gptq(W, None, 4, 16, 32, H=np.eye(64) * 2.0, n=1, sym=True)
    t = ref.rtn(W, 4, 16, sym=True)
    assert np.array_equal(r.quant.codes, t.codes)
    assert np.all(r.quant.zeros == 8)


@pytest.mark.parametrize("act", [False, True])
def test_static_groups_take_original_column_grids(act):
    """Static groups: every group's grid is the min/max grid of g consecutive original columns of the
    original weights, g_idx is k // g, and the stored layer dequantizes to the loop's weights."""
    rng = np.random.default_rng(29)
    d, g = 64, 16
    X = _correlated_x(rng, 96, d) * rng.uniform(0.3, 3.0, d)[None, :]
    W = rng.standard_normal((10, d)) * 0.02
    r = ref.gptq(W, [X], 4, g, 32, act_order=act, static_groups=True)
    q = r.quant
    for G in range(d // g):
        wg = W[:, G * g:(G + 1) * g]
        s_want = np.maximum(wg.max(1) - wg.min(1), 1e-8) / 15
        assert np.allclose(q.scales[:, G], s_want, rtol=1e-14)
        assert np.array_equal(q.zeros[:, G], np.rint((-wg.min(1)).astype(np.float32) / s_want.astype(np.float32)))
    assert np.array_equal(q.g_idx, np.arange(d) // g)
    assert np.array_equal(ref.dequantize(ref.pack(q.codes, 4), q.scales, q.zeros, q.g_idx, d), q.Q)
    r1 = ref.gptq(W, [X], 4, g, 1, act_order=act, static_groups=True)
    assert np.array_equal(r1.quant.codes, q.codes)          # blocked == unblocked


def test_static_groups_identity_hessian_is_original_order_rtn():
    """With H = I and act-order, static groups reduce to round-to-nearest over groups of consecutive
    original columns (dynamic groups would instead group consecutive processing positions)."""
    rng = np.random.default_rng(31)
    d = 64
    W = rng.standard_normal((8, d)) * 0.02
    H = np.diag(rng.uniform(1.0, 3.0, d)) * 2.0
    r = ref.gptq(W, None, 4, 16, 32, H=H, n=1, act_order=True, static_groups=True)
    assert np.array_equal(r.quant.codes, ref.rtn(W, 4, 16).codes)
    rd = ref.gptq(W, None, 4, 16, 32, H=H, n=1, act_order=True)
    assert np.array_equal(rd.quant.codes, ref.rtn(W, 4, 16, perm=rd.quant.perm).codes)


# ---------------------------------------------------------------- storage layouts

@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 6, 7, 8])
def test_dense_stream_is_positional_notation(bits):
    """A row's dense stream, read as one little-endian integer, is the row's codes as the digits of a
    number in base 2^bits (code k is digit k)."""
    rng = np.random.default_rng(bits)
    d = 96
    c = rng.integers(0, 1 << bits, size=(3, d)).astype(np.uint8)
    p = ref.pack_dense(c, bits).view(np.uint32)
    assert p.shape == (3, d * bits // 32)
    for r in range(3):
        value = sum(int(w) << (32 * i) for i, w in enumerate(p[r]))
        assert value == sum(int(c[r, k]) << (bits * k) for k in range(d))
    assert np.array_equal(ref.unpack_dense(ref.pack_dense(c, bits), d, bits), c)


@pytest.mark.parametrize("bits", [4, 8])
def test_dense_stream_equals_field_layout_at_full_fields(bits):
    """At 4 and 8 bits a code fills its field exactly, so the dense stream and pack() agree."""
    rng = np.random.default_rng(40 + bits)
    c = rng.integers(0, 1 << bits, size=(5, 64)).astype(np.uint8)
    assert np.array_equal(ref.pack_dense(c, bits), ref.pack(c, bits))


def test_byte_fields_closed_form():
    """Four 8-bit codes per word: column 4k + t in bits 8t .. 8t + 7 of word k."""
    c = np.array([[0x11, 0x22, 0x33, 0x44, 0xFF, 0x00, 0x80, 0x01]], np.uint8)
    p = ref.pack(c, 8).view(np.uint32)
    assert p.tolist() == [[0x44332211, 0x018000FF]]
    assert np.array_equal(ref.unpack(ref.pack(c, 8), 8, 8), c)
    assert ref.pack(c[:, :8] & 0x1F, 5).view(np.uint32)[0, 0] == 0x04130211    # 5-bit codes, byte fields


def test_dense_three_bit_saves_a_quarter():
    """Three-bit codes: 32 codes in 3 words, against 4 words in nibbles (tools page, Memory arithmetic:
    storage follows the bit width)."""
    c = np.zeros((1, 256), np.uint8)
    assert ref.pack_dense(c, 3).shape[1] == 24 and ref.pack(c, 3).shape[1] == 32


# ---------------------------------------------------------------- compact metadata

def test_compact_metadata_bits_per_weight():
    """Tools page, 'Memory arithmetic': 4-bit weights with a 16-bit scale and a 4-bit zero per group of
    128 cost about 0.16 extra bits per weight; groups of 32 cost about four times as much."""
    e = GOLD["memory_arithmetic"]
    over = ref.bits_per_weight(e["bits"], e["group_size"], e["scale_bits"], e["zero_bits"]) - e["bits"]
    assert over == pytest.approx(e["overhead_bits_per_weight_about"], abs=0.01)
    assert ref.bits_per_weight(4, 32, 16, 4) - 4 == pytest.approx(4 * over)


def test_compact_grid_closed_form():
    """A compact grid holds exactly what 16 bits of scale and a code-width zero can store, and the
    codes come from that stored grid."""
    wg = np.array([[-0.3, 0.7, 0.1], [0.5, 0.9, 0.6], [-0.9, -0.2, -0.5], [1e-12, 1e-12, 1e-12]])
    s, z = ref.group_grid(wg, 15, compact=True)
    s_exact = np.array([1.0, 0.4, 0.7, 1e-8]) / 15
    assert np.array_equal(s[:3], s_exact[:3].astype(np.float32).astype(np.float16).astype(np.float64))
    assert s[3] == 2.0 ** -24                      # below float16 range: the smallest subnormal
    assert z[0] == np.rint(0.3 / s[0]) and z[1] == 0 and z[2] == 15   # one-signed rows clamp
    q, dq = ref.quantize_to_grid(wg[:, :1], s[:, None], z[:, None], 15)
    assert np.allclose(dq[:, 0], s * (q[:, 0] - z))


@pytest.mark.parametrize("act,static,sym", [(False, False, False), (True, False, False), (True, True, False),
                                            (False, False, True)])
def test_compact_layer_stores_what_it_used(act, static, sym):
    rng = np.random.default_rng(37)
    d = 64
    X = _correlated_x(rng, 96, d) * rng.uniform(0.3, 3.0, d)[None, :]
    W = rng.standard_normal((10, d)) * 0.02
    W[0] += 0.08                                   # positive row: zeros clamp at 0
    r = ref.gptq(W, [X], 4, 16, 32, act_order=act, static_groups=static, sym=sym, compact=True)
    q = r.quant
    assert np.array_equal(q.scales, q.scales.astype(np.float16).astype(np.float64))
    assert q.zeros.min() >= 0 and q.zeros.max() <= 15
    assert np.array_equal(ref.dequantize(ref.pack(q.codes, 4), q.scales.astype(np.float16).astype(np.float64),
                                         q.zeros, q.g_idx, d), q.Q)
    r1 = ref.gptq(W, [X], 4, 16, 1, act_order=act, static_groups=static, sym=sym, compact=True)
    assert np.array_equal(r1.quant.codes, q.codes)
