"""Float64 CPU oracle of the GPTQ single-layer solver.

TEST INFRASTRUCTURE. Only the test suite, the smoke check in __graft_entry__ and the CPU-baseline
leg of bench.py may import this module. The product path (the HIP library and its Python binding)
never imports, links or runs anything here, and this module imports nothing from the product.

It is a plain, slow, step-by-step statement of what the solver computes, written from these pages:

* GPTQ tools page (ozercemkelahmet.com/tools/gptq), "How it works", Steps 3-8, "Optional
  refinements" and the section "A minimal Python sketch" (the sketch is read as a description of
  the computation, not transcribed). Step 8 also gives the inference use of the stored layer
  (unpack, scale, multiply), stated here as dequantize / dequant_matmul.
* "GPTQ Quantization: Complete Technical Guide" (notes.jayaprakash.net), sections "Quantization
  Equation", "Example: Quantizing a Single Weight", "Computing the Hessian", "Damping Factor".
* "Paper breakdown: GPTQ" (ai360xpert.com), "How It Works" (lazy batching).
* "What Is GPTQ? Classic 4-Bit LLM Quantization" (ai-tldr.dev), "How it works", Step 3 (groups).

Arithmetic is float64 throughout (inputs are upcast exactly), with one exception: the two
rounding decisions (a code from w / scale, a zero point from -wmin / scale) divide in float32. The
tools page's sketch converts the weights to float32 before its loop, so its w / scale and
-wmin / scale are float32 divisions of float32 values; the oracle takes those two quotients the same
way, from its float64 operands rounded to float32, and keeps float64 everywhere else.
Dense algebra uses library primitives: BLAS matrix products and the LAPACK Cholesky routines
(potrf / potri) that the sketch's cholesky / cholesky_inverse / cholesky(upper) calls name.

Readings taken where the pages are silent, garbled or disagree:

* H is accumulated as the sum over token chunks of 2 X_c^T X_c and normalised by the token count
  n before damping (the sketch's 2 X^T X / n).
* Damping adds damp * mean(diag(H/n)) to the diagonal (tools page Step 4 and the sketch), not
  damp * trace(H) (Technical Guide, "Damping Factor").
* Grids are asymmetric min/max grids with unsigned codes in [0, 2^bits - 1]; a group is g
  consecutive columns of one row in processing order; group_size <= 0 means one group per row.
* A symmetric grid is the same min/max recipe on [-max|w|, max|w|] with the zero fixed at the middle
  code 2^(bits - 1) (the Technical Guide's signed int4 range [-8, 7] as unsigned codes).
* A group's grid is computed from the current (error-updated) weights at the group's first column;
  with static groups, from the original weights of g consecutive original columns, before the loop.
* Blocks and groups must nest (B % g == 0 or g % B == 0); the last block and last group may be short.
* Act-order processes columns by descending diag(H); ties keep the lower original index first.
* Rounding is round-half-to-even (numpy rint), as torch.round in the sketch.

Parity unpinned (no example on the pages fixes them; they rest on the readings above): the moment a
group grid is taken when g < d, the act-order tie-break, the symmetric grid's scale (the pages give
its code range and value = code x scale, not how the scale is chosen) and what static groups mean
(the pages give only the setting's name).
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Iterable, Optional, Tuple

import numpy as np
from scipy.linalg import lapack


class NotPositiveDefinite(ArithmeticError):
    """The damped Hessian has a non-positive pivot (1-based index `pivot`, LAPACK convention)."""

    def __init__(self, pivot: int):
        super().__init__(f"leading minor {pivot} is not positive definite")
        self.pivot = int(pivot)


# --------------------------------------------------------------------------------------------
# Hessian, damping, ordering, factor  (tools page Steps 3, 4, 6; sketch; "Optional refinements")
# --------------------------------------------------------------------------------------------

def hessian(chunks: Iterable[np.ndarray]) -> Tuple[np.ndarray, int]:
    """Unnormalised Hessian sum over token chunks: sum_c 2 X_c^T X_c, and the token count n.

    Each X_c is (tokens x d). The layer Hessian is proportional to X X^T in the pages' feature-major
    notation (tools page, Step 3); the sketch forms 2 X^T X / n with X = (samples x features), and
    the Technical Guide ("Computing the Hessian") sums outer products and then averages.
    """
    H = None
    n = 0
    for xc in chunks:
        x = np.asarray(xc, dtype=np.float64)
        if H is None:
            H = np.zeros((x.shape[1], x.shape[1]), dtype=np.float64)
        H += 2.0 * (x.T @ x)
        n += x.shape[0]
    if H is None:
        raise ValueError("no calibration chunks")
    return H, n


def act_order_perm(H: np.ndarray) -> np.ndarray:
    """Processing order for act-order: columns by descending diag(H), ties by lower index first.

    Tools page, "Optional refinements", Act-order.
    """
    diag = np.diag(H)
    return np.argsort(-diag, kind="stable").astype(np.int64)


def damp_and_order(H: np.ndarray, n: int, damp: float, act_order: bool,
                   perm: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray, float]:
    """Normalise, damp and (optionally) reorder: Hhat = (H/n + lam I)[perm][:, perm].

    lam = damp * mean(diag(H/n)) (tools page, Step 4: about one percent of the average diagonal).
    `perm` may be given to impose a processing order (a test uses it to follow another
    implementation's order among keys equal within rounding); otherwise it is act_order_perm(H)
    when act_order is set and the identity when not.
    """
    d = H.shape[0]
    Hn = np.asarray(H, dtype=np.float64) / float(n)
    mean_diag = float(np.mean(np.diag(Hn)))
    if not (mean_diag > 0.0):
        raise ValueError("mean of diag(H) must be positive")
    lam = float(damp) * mean_diag
    Hd = Hn + lam * np.eye(d)
    if perm is None:
        perm = act_order_perm(H) if act_order else np.arange(d, dtype=np.int64)
    perm = np.asarray(perm, dtype=np.int64)
    return Hd[np.ix_(perm, perm)], perm, lam


def inverse_cholesky_upper(Hhat: np.ndarray) -> np.ndarray:
    """U: the upper Cholesky factor of Hhat^-1, so that Hhat^-1 = U^T U.

    Tools page, Step 6 (the Cholesky factor of the inverse Hessian is computed once) and the
    sketch's three calls: the Cholesky factor of Hhat, the inverse from that factor, then the
    upper Cholesky factor of the inverse. Raises NotPositiveDefinite with the failing pivot.
    """
    c, info = lapack.dpotrf(np.asarray(Hhat, dtype=np.float64), lower=1, clean=1)
    if info > 0:
        raise NotPositiveDefinite(info)
    if info < 0:
        raise ValueError(f"dpotrf argument {-info}")
    inv, info = lapack.dpotri(c, lower=1)
    if info != 0:
        raise NotPositiveDefinite(info)
    inv = np.tril(inv) + np.tril(inv, -1).T
    u, info = lapack.dpotrf(inv, lower=0, clean=1)
    if info != 0:
        raise NotPositiveDefinite(info)
    return np.triu(u)


# --------------------------------------------------------------------------------------------
# The grid  (sketch's quantize_to_grid and its per-row min/max grid; Technical Guide,
# "Quantization Equation"; What Is GPTQ?, Step 3 for groups)
# --------------------------------------------------------------------------------------------

def _round_ratio(num: np.ndarray, den: np.ndarray) -> np.ndarray:
    """rint(num / den) with the division taken in float32 (the decision precision)."""
    return np.rint(np.asarray(num, dtype=np.float32) / np.asarray(den, dtype=np.float32)).astype(np.float64)


def _ratio32(num, den) -> np.ndarray:
    return (np.asarray(num, dtype=np.float32) / np.asarray(den, dtype=np.float32)).astype(np.float64)


FP16_MIN_SUB = 2.0 ** -24      # smallest positive float16
FP16_MAX = 65504.0


def fp16_scale(scale32: np.ndarray) -> np.ndarray:
    """The scale as stored in 16 bits: the float32 scale rounded to the nearest float16 (ties to
    even), kept positive and finite (a scale below half the smallest subnormal takes that subnormal,
    one above the largest finite float16 takes that)."""
    s = np.asarray(scale32, dtype=np.float32).astype(np.float16).astype(np.float64)
    return np.clip(np.where(s == 0.0, FP16_MIN_SUB, s), FP16_MIN_SUB, FP16_MAX)


def group_grid(wg: np.ndarray, maxq: int, sym: bool = False, compact: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    """Min/max grid of each row of wg (rows x columns of one group).

    Asymmetric (the sketch): scale = max(wmax - wmin, 1e-8) / maxq and zero = round(-wmin / scale).
    Symmetric (tools page, "Optional refinements", grids without a zero point to fit; the Technical
    Guide's int4 range [-8, 7] with value = code x scale): the same recipe on the range [-m, m],
    m = max(|wmin|, |wmax|), so scale = max(2 m, 1e-8) / maxq, with the zero fixed at the middle code
    (maxq + 1) / 2 = 2^(bits - 1), which turns the signed range into unsigned codes [0, maxq].
    """
    wmin = np.min(wg, axis=1)
    wmax = np.max(wg, axis=1)
    if sym:
        m = np.maximum(np.abs(wmin), np.abs(wmax))
        scale = np.maximum(2.0 * m, 1e-8) / float(maxq)
        if compact:
            scale = fp16_scale(_scale32(2.0 * m, maxq))
        return scale, np.full(scale.shape, float((maxq + 1) // 2))
    scale = np.maximum(wmax - wmin, 1e-8) / float(maxq)
    if compact:
        scale = fp16_scale(_scale32(wmax - wmin, maxq))
        return scale, np.clip(_round_ratio(-wmin, scale), 0.0, float(maxq))
    zero = _round_ratio(-wmin, scale)
    return scale, zero


def _scale32(span: np.ndarray, maxq: int) -> np.ndarray:
    """max(span, 1e-8) / maxq in float32, the precision in which the scale's 16-bit rounding is decided."""
    sp = np.maximum(np.asarray(span, dtype=np.float32), np.float32(1e-8))
    return (sp / np.float32(maxq)).astype(np.float64)


def quantize_to_grid(w: np.ndarray, scale: np.ndarray, zero: np.ndarray, maxq: int) -> Tuple[np.ndarray, np.ndarray]:
    """Code q = clamp(round(w / scale) + zero, 0, maxq) and its value scale * (q - zero)."""
    q = np.clip(_round_ratio(w, scale) + zero, 0.0, float(maxq))
    return q, scale * (q - zero)


# --------------------------------------------------------------------------------------------
# The column loop with lazy blocks  (tools page Steps 5, 7, 8; Paper breakdown "How It Works")
# --------------------------------------------------------------------------------------------

@dataclass
class QuantResult:
    codes: np.ndarray       # uint8 rows x d, original column order
    scales: np.ndarray      # float64 rows x ngroups (groups in processing order)
    zeros: np.ndarray       # int32 rows x ngroups
    g_idx: np.ndarray       # int32 d: group of each original column
    perm: np.ndarray        # int64 d: processing order (perm[j] = original column processed j-th)
    loss: float             # sum over rows and columns of err^2
    row_loss: np.ndarray    # float64 rows
    Q: np.ndarray           # float64 rows x d dequantised weights, original column order
    codes_proc: np.ndarray  # uint8 rows x d, processing order
    w_seen: Optional[np.ndarray] = None  # rows x d, processing order: each weight when it was quantized
    adopted: int = 0        # follow mode: tie-window decisions taken from the followed result
    adopted_diff: int = 0   # ... of which differ from this oracle's own choice
    near_ties: int = 0      # decisions whose ratio lay inside the tie window
    extra: dict = field(default_factory=dict)


def check_geometry(d: int, group_size: int, block_size: int) -> int:
    """Effective group size; raises ValueError for shapes the solver rejects."""
    if d <= 0:
        raise ValueError("d must be positive")
    g = d if group_size <= 0 else int(group_size)
    if g == 1:
        raise ValueError("group_size 1 is rejected (Technical Guide, Don'ts: group_size=1 will fail)")
    if block_size <= 0:
        raise ValueError("block_size must be positive")
    if g < d and not (block_size % g == 0 or g % block_size == 0):
        raise ValueError("block_size and group_size must nest")
    return g


def _follow_pick(own: np.ndarray, ratio: np.ndarray, offset: np.ndarray, lo: float, hi: float,
                 other: Optional[np.ndarray], tau: float):
    """Take `other` where ratio lies within tau of a half-integer and other is a neighbour choice."""
    frac = ratio - np.floor(ratio)
    tie = np.abs(frac - 0.5) < tau
    if other is None or not np.any(tie):
        return own, 0, 0, int(np.count_nonzero(tie))
    c1 = np.clip(np.floor(ratio) + offset, lo, hi)
    c2 = np.clip(np.ceil(ratio) + offset, lo, hi)
    ok = tie & ((other == c1) | (other == c2))
    out = np.where(ok, other, own)
    return out, int(np.count_nonzero(ok)), int(np.count_nonzero(ok & (other != own))), int(np.count_nonzero(tie))


def _follow_scale(own: np.ndarray, s32: np.ndarray, other: Optional[np.ndarray], rtol: float = 1e-5):
    """Compact grids: take the other implementation's 16-bit scale where this oracle's float32 scale
    lies within rtol of a float16 rounding boundary and the other scale is one of the two neighbours."""
    if other is None:
        return own, 0
    lo = fp16_scale(s32 * (1.0 - rtol))
    hi = fp16_scale(s32 * (1.0 + rtol))
    other = np.asarray(other, dtype=np.float64)
    ok = (lo != hi) & ((other == lo) | (other == hi))
    return np.where(ok, other, own), int(np.count_nonzero(ok & (other != own)))


def quantize_layer(W: np.ndarray, U: np.ndarray, bits: int, group_size: int, block_size: int,
                   perm: Optional[np.ndarray] = None, grid: Optional[Tuple[np.ndarray, np.ndarray]] = None,
                   follow: Optional[Tuple[np.ndarray, ...]] = None, tau: float = 1e-3,
                   sym: bool = False, static_groups: bool = False, compact: bool = False) -> QuantResult:
    """Quantize W (rows x d, original column order) with U (upper, processing order).

    For each block of B columns in processing order, and each column i in it:
      * at a group's first column, the group grid comes from the current weights of its columns;
      * q = clamp(round(w/s) + z, 0, maxq); err = (w - s (q - z)) / U[i, i]   (Step 5, parts 1-3);
      * the columns after i inside the block take -err * U[i, j] at once       (Step 5, part 4);
      * the block's errors are kept and, at block end, the columns after the block take
        -Err @ U[block, after] in one product                                  (Step 7, lazy batch).
    Step 8: one (scale, zero) per group; codes are returned in the original column order with g_idx.

    grid: optional fixed (scales, zeros), rows x ngroups, used instead of min/max grids.
    sym: symmetric grids (see group_grid).
    static_groups: every group's grid is fixed before the loop from the original weights of g
    consecutive original columns (the Technical Guide's static_groups setting; the pages give only
    its name, so this plain reading of "static" is parity-unpinned); column i then uses the grid of
    group perm[i] // g, and g_idx is k // g whatever the order.
    compact: each grid is stored as a 16-bit scale and a zero of the code width (tools page, "Memory
    arithmetic"), and the loop quantizes with exactly those: the scale rounded to float16 (see
    fp16_scale), the zero clamped to [0, maxq]. With follow=(codes, zeros, scales) the oracle takes
    the other side's float16 scale where its own float32 scale sits on a rounding boundary.
    follow: optional (codes, zeros) of another implementation in processing order; at decisions whose
    float32 ratio lies within `tau` of a half-integer this oracle takes that implementation's choice
    when it is one of the two nearest grid points (both are correct roundings within the tie window).
    """
    W = np.asarray(W, dtype=np.float64)
    rows, d = W.shape
    U = np.asarray(U)            # float64, or float32 (each block's rows are upcast exactly when used)
    if U.shape != (d, d):
        raise ValueError("U shape")
    g = check_geometry(d, group_size, block_size)
    B = int(block_size)
    maxq = (1 << int(bits)) - 1
    ngroups = (d + g - 1) // g
    perm = np.arange(d, dtype=np.int64) if perm is None else np.asarray(perm, dtype=np.int64)

    Wp = W[:, perm].copy()                      # working copy, processing order
    codes_p = np.zeros((rows, d), dtype=np.float64)
    Qp = np.zeros((rows, d), dtype=np.float64)
    seen = np.zeros((rows, d), dtype=np.float64)
    scales = np.zeros((rows, ngroups), dtype=np.float64)
    zeros = np.zeros((rows, ngroups), dtype=np.float64)
    row_loss = np.zeros(rows, dtype=np.float64)
    f_codes = None if follow is None else np.asarray(follow[0], dtype=np.float64)
    f_zeros = None if follow is None else np.asarray(follow[1], dtype=np.float64)
    f_scales = None if (follow is None or len(follow) < 3) else np.asarray(follow[2], dtype=np.float64)

    def grid_of(wg, gi):
        """A group's grid from its current weights wg, following the other side at ties."""
        nonlocal adopted, adopted_diff, near
        sg, zg = group_grid(wg, maxq, sym, compact)
        wmin = np.min(wg, axis=1)
        if compact and f_scales is not None:
            span = 2.0 * np.maximum(np.abs(wmin), np.abs(np.max(wg, axis=1))) if sym else np.max(wg, axis=1) - wmin
            sg, ad = _follow_scale(sg, _scale32(span, maxq), f_scales[:, gi])
            adopted_diff += ad
            if not sym:
                zg = np.clip(_round_ratio(-wmin, sg), 0.0, float(maxq))
        if f_zeros is not None and not sym:
            lo, hi = (0.0, float(maxq)) if compact else (-np.inf, np.inf)
            zg, a, ad, nt = _follow_pick(zg, _ratio32(-wmin, sg), np.zeros(len(zg)), lo, hi, f_zeros[:, gi], tau)
            adopted += a
            adopted_diff += ad
            near += nt
        return sg, zg
    adopted = adopted_diff = near = 0

    if static_groups and grid is None:
        for gi in range(ngroups):
            cols = slice(gi * g, min((gi + 1) * g, d))
            scales[:, gi], zeros[:, gi] = grid_of(W[:, cols], gi)

    s = z = None
    for b in range(0, d, B):
        e_blk = min(b + B, d)
        Ub = np.asarray(U[b:e_blk], dtype=np.float64)     # the block's rows of U: Ub[i - b] is U[i]
        Err = np.zeros((rows, e_blk - b), dtype=np.float64)
        for i in range(b, e_blk):
            if static_groups and grid is None:
                s = scales[:, perm[i] // g]
                z = zeros[:, perm[i] // g]
            elif i % g == 0:
                gi = i // g
                if grid is not None:
                    s = np.asarray(grid[0], dtype=np.float64)[:, gi]
                    z = np.asarray(grid[1], dtype=np.float64)[:, gi]
                else:
                    s, z = grid_of(Wp[:, i:min(i + g, d)], gi)
                scales[:, gi] = s
                zeros[:, gi] = z
            w = Wp[:, i].copy()
            seen[:, i] = w
            q, dq = quantize_to_grid(w, s, z, maxq)
            if f_codes is not None:
                q2, a, ad, nt = _follow_pick(q, _ratio32(w, s), z, 0.0, float(maxq), f_codes[:, i], tau)
                if a:
                    q = q2
                    dq = s * (q - z)
                adopted += a
                adopted_diff += ad
                near += nt
            codes_p[:, i] = q
            Qp[:, i] = dq
            err = (w - dq) / Ub[i - b, i]
            Err[:, i - b] = err
            row_loss += err * err
            if i + 1 < e_blk:
                Wp[:, i + 1:e_blk] -= np.outer(err, Ub[i - b, i + 1:e_blk])
        if e_blk < d:
            Wp[:, e_blk:] -= Err @ Ub[:, e_blk:]

    codes = np.zeros((rows, d), dtype=np.uint8)
    codes[:, perm] = codes_p.astype(np.uint8)
    Q = np.zeros((rows, d), dtype=np.float64)
    Q[:, perm] = Qp
    g_idx = np.zeros(d, dtype=np.int32)
    if static_groups:
        g_idx[:] = (np.arange(d) // g).astype(np.int32)
    else:
        g_idx[perm] = (np.arange(d) // g).astype(np.int32)
    return QuantResult(codes=codes, scales=scales, zeros=zeros.astype(np.int32), g_idx=g_idx, perm=perm,
                       loss=float(np.sum(row_loss)), row_loss=row_loss, Q=Q,
                       codes_proc=codes_p.astype(np.uint8), w_seen=seen, adopted=adopted, adopted_diff=adopted_diff,
                       near_ties=near)


# --------------------------------------------------------------------------------------------
# Packing  (tools page, Step 8: eight 4-bit codes per 32-bit word)
# --------------------------------------------------------------------------------------------

def field_bits(bits: int) -> int:
    """Width of the field pack() gives a code: a nibble for up to 4 bits, a byte for 5 to 8."""
    if not (1 <= bits <= 8):
        raise ValueError("codes have 1 to 8 bits")
    return 4 if bits <= 4 else 8


def pack(codes: np.ndarray, bits: int) -> np.ndarray:
    """int32 words of fixed fields along each row: with f = field_bits(bits), field t (bits f t ..
    f t + f - 1) of word k holds column (32 / f) k + t, so eight 4-bit codes per word (tools page,
    Step 8) or four 8-bit codes."""
    c = np.asarray(codes)
    rows, d = c.shape
    f = field_bits(bits)
    per = 32 // f
    if d % per != 0:
        raise ValueError(f"d must be a multiple of {per}")
    if np.any(c.astype(np.int64) >= (1 << bits)) or np.any(c.astype(np.int64) < 0):
        raise ValueError("code out of range")
    words = np.zeros((rows, d // per), dtype=np.uint64)
    for t in range(per):
        words |= c[:, t::per].astype(np.uint64) << np.uint64(f * t)
    return words.astype(np.uint32).view(np.int32)


def unpack(packed: np.ndarray, d: int, bits: int = 4) -> np.ndarray:
    """Inverse of pack."""
    f = field_bits(bits)
    per = 32 // f
    p = np.asarray(packed).view(np.uint32).astype(np.uint64)
    out = np.zeros((p.shape[0], d), dtype=np.uint8)
    for t in range(per):
        out[:, t::per] = ((p >> np.uint64(f * t)) & np.uint64((1 << f) - 1)).astype(np.uint8)
    return out


def pack_dense(codes: np.ndarray, bits: int) -> np.ndarray:
    """Each row as one little-endian bit stream of exactly `bits` bits per code: code k takes stream
    bits bits k .. bits k + bits - 1, and stream bit t is bit t % 32 of word t // 32 (so 32 three-bit
    codes fill three words). Needs d * bits to be a multiple of 32."""
    c = np.asarray(codes).astype(np.int64)
    rows, d = c.shape
    if not (1 <= bits <= 8) or (d * bits) % 32 != 0:
        raise ValueError("bits in 1..8 and d * bits a multiple of 32")
    if np.any(c >= (1 << bits)) or np.any(c < 0):
        raise ValueError("code out of range")
    nw = d * bits // 32
    words = np.zeros((rows, nw), dtype=np.uint64)
    for k in range(d):
        pos = k * bits
        w, sh = pos // 32, pos % 32
        v = c[:, k].astype(np.uint64) << np.uint64(sh)          # up to 39 bits
        words[:, w] |= v & np.uint64(0xFFFFFFFF)
        if sh + bits > 32:
            words[:, w + 1] |= v >> np.uint64(32)
    return words.astype(np.uint32).view(np.int32)


def unpack_dense(packed: np.ndarray, d: int, bits: int) -> np.ndarray:
    """Inverse of pack_dense."""
    p = np.asarray(packed).view(np.uint32).astype(np.uint64)
    out = np.zeros((p.shape[0], d), dtype=np.uint8)
    for k in range(d):
        pos = k * bits
        w, sh = pos // 32, pos % 32
        v = p[:, w] >> np.uint64(sh)
        if sh + bits > 32:
            v |= p[:, w + 1] << np.uint64(32 - sh)
        out[:, k] = (v & np.uint64((1 << bits) - 1)).astype(np.uint8)
    return out


# --------------------------------------------------------------------------------------------
# Using the stored layer  (tools page Step 8: at inference a kernel unpacks, scales and multiplies;
# What Is GPTQ, "How it works": each group is expanded back to higher precision for the product)
# --------------------------------------------------------------------------------------------

def dequantize(packed: np.ndarray, scales: np.ndarray, zeros: np.ndarray, g_idx: np.ndarray,
               d: int, bits: int = 4, dense: bool = False) -> np.ndarray:
    """Weights rows x d, original column order: column j of row r is
    scales[r, g] * (code[r, j] - zeros[r, g]) with g = g_idx[j], the group column j was quantized in.
    `packed` is in pack()'s layout, or pack_dense()'s with dense=True."""
    codes = (unpack_dense(packed, d, bits) if dense else unpack(packed, d, bits)).astype(np.float64)
    g = np.asarray(g_idx, dtype=np.int64)
    s = np.asarray(scales, dtype=np.float64)[:, g]
    z = np.asarray(zeros, dtype=np.float64)[:, g]
    return s * (codes - z)


def dequant_matmul(x: np.ndarray, packed: np.ndarray, scales: np.ndarray, zeros: np.ndarray,
                   g_idx: np.ndarray, d: int, bits: int = 4, dense: bool = False) -> np.ndarray:
    """The layer's output y = x W^T (m x rows) for inputs x (m x d), W the dequantized weights."""
    W = dequantize(packed, scales, zeros, g_idx, d, bits, dense)
    return np.asarray(x, dtype=np.float64) @ W.T


def bits_per_weight(bits: int, group_size: int, scale_bits: int = 16, zero_bits: int = 4) -> float:
    """Storage cost per weight with one scale and zero per group (tools page, "Memory arithmetic")."""
    return bits + (scale_bits + zero_bits) / float(group_size)


# --------------------------------------------------------------------------------------------
# Whole layer, baselines and the objective
# --------------------------------------------------------------------------------------------

@dataclass
class LayerResult:
    H: np.ndarray
    n: int
    Hhat: np.ndarray
    lam: float
    U: np.ndarray
    quant: QuantResult
    packed: Optional[np.ndarray]


def gptq(W: np.ndarray, chunks: Iterable[np.ndarray], bits: int, group_size: int, block_size: int,
         act_order: bool = False, damp: float = 0.01, perm: Optional[np.ndarray] = None,
         follow: Optional[Tuple[np.ndarray, np.ndarray]] = None, tau: float = 1e-3,
         H: Optional[np.ndarray] = None, n: Optional[int] = None, sym: bool = False,
         static_groups: bool = False, compact: bool = False) -> LayerResult:
    """The whole single-layer solver: Hessian, damping and order, factor, column loop, packing."""
    if H is None:
        H, n = hessian(chunks)
    Hhat, p, lam = damp_and_order(H, n, damp, act_order, perm)
    U = inverse_cholesky_upper(Hhat)
    qr = quantize_layer(W, U, bits, group_size, block_size, perm=p, follow=follow, tau=tau, sym=sym,
                        static_groups=static_groups, compact=compact)
    d = qr.codes.shape[1]
    packed = pack(qr.codes, bits) if d % (32 // field_bits(bits)) == 0 else None
    return LayerResult(H=H, n=n, Hhat=Hhat, lam=lam, U=U, quant=qr, packed=packed)


def rtn(W: np.ndarray, bits: int, group_size: int, perm: Optional[np.ndarray] = None,
        sym: bool = False) -> QuantResult:
    """Round-to-nearest baseline: the same grids, taken from the unmodified weights, no feedback."""
    W = np.asarray(W, dtype=np.float64)
    rows, d = W.shape
    g = d if group_size <= 0 else int(group_size)
    maxq = (1 << int(bits)) - 1
    perm = np.arange(d, dtype=np.int64) if perm is None else np.asarray(perm, dtype=np.int64)
    Wp = W[:, perm]
    ngroups = (d + g - 1) // g
    codes_p = np.zeros((rows, d))
    Qp = np.zeros((rows, d))
    scales = np.zeros((rows, ngroups))
    zeros = np.zeros((rows, ngroups))
    for gi in range(ngroups):
        sl = slice(gi * g, min((gi + 1) * g, d))
        s, z = group_grid(Wp[:, sl], maxq, sym)
        q, dq = quantize_to_grid(Wp[:, sl], s[:, None], z[:, None], maxq)
        codes_p[:, sl] = q
        Qp[:, sl] = dq
        scales[:, gi] = s
        zeros[:, gi] = z
    codes = np.zeros((rows, d), dtype=np.uint8)
    codes[:, perm] = codes_p.astype(np.uint8)
    Q = np.zeros((rows, d))
    Q[:, perm] = Qp
    g_idx = np.zeros(d, dtype=np.int32)
    g_idx[perm] = (np.arange(d) // g).astype(np.int32)
    return QuantResult(codes=codes, scales=scales, zeros=zeros.astype(np.int32), g_idx=g_idx, perm=perm,
                       loss=float("nan"), row_loss=np.full(rows, np.nan), Q=Q, codes_proc=codes_p.astype(np.uint8))


def objective(W: np.ndarray, Q: np.ndarray, Hhat: np.ndarray) -> float:
    """sum over rows of (W - Q)_r Hhat (W - Q)_r^T (tools page, Step 2, with the damped Hessian).

    W, Q and Hhat must be in the same column order.
    """
    D = np.asarray(W, dtype=np.float64) - np.asarray(Q, dtype=np.float64)
    return float(np.sum((D @ Hhat) * D))


def brute_force(W: np.ndarray, Hhat: np.ndarray, bits: int) -> Tuple[float, np.ndarray]:
    """Exhaustive minimum of the objective over each row's grid (one group per row; tiny d only)."""
    W = np.asarray(W, dtype=np.float64)
    rows, d = W.shape
    if d > 8:
        raise ValueError("brute force is for d <= 8")
    maxq = (1 << int(bits)) - 1
    s, z = group_grid(W, maxq)
    grids = np.stack(np.meshgrid(*([np.arange(maxq + 1, dtype=np.float64)] * d), indexing="ij"), -1).reshape(-1, d)
    best = 0.0
    bestQ = np.zeros_like(W)
    for r in range(rows):
        dq = s[r] * (grids - z[r])
        D = W[r][None, :] - dq
        f = np.sum((D @ Hhat) * D, axis=1)
        k = int(np.argmin(f))
        best += float(f[k])
        bestQ[r] = dq[k]
    return best, bestQ
