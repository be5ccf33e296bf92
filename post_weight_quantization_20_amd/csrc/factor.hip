// Damping, act-order and the upper Cholesky factor U of the damped inverse Hessian (Hhat^-1 = U^T U).
//
// GPTQ tools page, "How it works", Step 4 (damping: a small multiple of the mean diagonal is added
// to the diagonal), "Optional refinements" (act-order: columns by descending diag(H)), and Step 6
// (the Cholesky factor of the inverse Hessian is computed once; its rows give every step's update).
//
// Route. With J the exchange matrix, if J Hhat J = L L^T (lower Cholesky) then Hhat = R R^T with
// R = J L J upper, and U = R^-1 = J L^-1 J. So the damped, permuted Hessian is gathered already
// reversed, factored by a blocked right-looking Cholesky, inverted in place by a blocked
// right-looking triangular inverse, and rotated back by 180 degrees. This takes 2/3 d^3 flops and
// never forms Hhat^-1 (the page's sketch takes the Cholesky factor of Hhat, forms the inverse from it
// and factors that again, 4/3 d^3 flops; both give the same U in exact arithmetic).
//
// Blocking (nb = 128): per diagonal block one workgroup factors the block in LDS and replaces it
// by the inverse of its Cholesky factor; every other product (panel solve, symmetric trailing
// update, the triangular-inverse products) is an fp32 MFMA GEMM on the whole device.
#include "common.hpp"

#include <cfloat>

namespace gptq {
namespace {

constexpr int NB = 128;

struct FactorWork {
  double* lam;     // damping added to the diagonal
  int64_t* info;   // 0, or the 1-based index of the first non-positive pivot
  int* status;     // 1 when mean(diag H) is not positive and finite
  float* keys;     // diag(H), the act-order sort key
};

// mean(diag(H)) / n * damp, in float64 and a fixed summation order; also copies diag(H).
__global__ __launch_bounds__(1024) void diag_stats_kernel(const float* __restrict__ H, int64_t d, int64_t n,
                                                          double damp, FactorWork w) {
  __shared__ double part[1024];
  double acc = 0.0;
  for (int64_t i = threadIdx.x; i < d; i += 1024) {
    const float h = H[i * d + i];
    w.keys[i] = h;
    acc += (double)h;
  }
  part[threadIdx.x] = acc;
  __syncthreads();
  for (int s = 512; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) part[threadIdx.x] += part[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double mean = part[0] / (double)d / (double)n;
    const bool ok = mean > 0.0 && mean < 1.0e300;
    *w.status = ok ? 0 : 1;
    *w.lam = ok ? damp * mean : 0.0;
    *w.info = 0;
  }
}

// perm[rank(i)] = i with rank = number of keys that sort before key i: larger keys first, equal
// keys by lower index first (a stable descending sort). NaN keys sort last.
__global__ __launch_bounds__(256) void rank_perm_kernel(const float* __restrict__ keys, int64_t d,
                                                        int32_t* __restrict__ perm) {
  __shared__ float tile[2048];
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  float ki = i < d ? keys[i] : 0.0f;
  if (ki != ki) ki = -INFINITY;
  int64_t rank = 0;
  for (int64_t t0 = 0; t0 < d; t0 += 2048) {
    const int64_t cnt = min<int64_t>(2048, d - t0);
    __syncthreads();
    for (int e = threadIdx.x; e < cnt; e += 256) {
      float v = keys[t0 + e];
      tile[e] = (v != v) ? -INFINITY : v;
    }
    __syncthreads();
    if (i < d) {
      for (int e = 0; e < cnt; ++e) {
        const float kj = tile[e];
        const int64_t j = t0 + e;
        rank += (kj > ki) || (kj == ki && j < i);
      }
    }
  }
  if (i < d) perm[rank] = (int32_t)i;
}

// dst[r][c] = src[r][c] for a rows x cols block (leading dimensions ldd, lds); stages the operand of a
// product whose output overwrites it. Unit `part` of `nparts` moves every nparts-th group of 256
// four-element row pieces, as 16-byte accesses when both sides allow it.
struct Copy2D {
  float* dst;
  const float* src;
  int64_t ldd, lds, rows, cols;
  int vec;
};

GPTQ_DEV void copy_part(const Copy2D& c, int64_t part, int64_t nparts) {
  const int64_t c4 = (c.cols + 3) / 4, total = c.rows * c4;
  for (int64_t i = part * 256 + threadIdx.x; i < total; i += nparts * 256) {
    const int64_t r = i / c4, col = (i % c4) * 4;
    if (c.vec && col + 4 <= c.cols) {
      *reinterpret_cast<float4*>(c.dst + r * c.ldd + col) = *reinterpret_cast<const float4*>(c.src + r * c.lds + col);
    } else {
      for (int64_t e = col; e < c.cols && e < col + 4; ++e) c.dst[r * c.ldd + e] = c.src[r * c.lds + e];
    }
  }
}

Copy2D make_copy(float* dst, int64_t ldd, const float* src, int64_t lds, int64_t rows, int64_t cols) {
  Copy2D c{dst, src, ldd, lds, std::max<int64_t>(rows, 0), std::max<int64_t>(cols, 0), 0};
  c.vec = (uintptr_t)dst % 16 == 0 && (uintptr_t)src % 16 == 0 && ldd % 4 == 0 && lds % 4 == 0;
  return c;
}

// Workgroups for a copy of `rows` x `cols` (one per 4096 four-element pieces, at most 1024).
unsigned copy_groups(int64_t rows, int64_t cols) {
  const int64_t pieces = std::max<int64_t>(rows, 0) * ((std::max<int64_t>(cols, 0) + 3) / 4);
  return (unsigned)std::min<int64_t>((pieces + 4095) / 4096, 1024);
}

// Two independent copies in one launch: blocks [0, g0) take the first, the rest the second.
__global__ __launch_bounds__(256) void copy2_kernel(Copy2D c0, Copy2D c1, unsigned g0) {
  if (blockIdx.x < g0) copy_part(c0, blockIdx.x, g0);
  else copy_part(c1, blockIdx.x - g0, gridDim.x - g0);
}

__global__ void iota_kernel(int32_t* perm, int64_t d) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < d) perm[i] = (int32_t)i;
}

// A[i][j] (j <= i) = Hhat[p(i)][p(j)], p(i) = perm[d-1-i]: the damped, normalised Hessian in
// processing order, reversed. H's upper triangle is authoritative. Off the diagonal this reads only
// H's strict upper triangle and writes only A's strict lower one; the diagonal comes from the copy
// diag_stats_kernel took (keys), so A may be H itself (the factor in place).
__global__ __launch_bounds__(256) void gather_kernel(const float* H, int64_t d, int64_t n,
                                                     const int32_t* __restrict__ perm, FactorWork w, float* A) {
  const int64_t i = blockIdx.x;
  const int64_t pi = perm[d - 1 - i];
  const double lam = *w.lam;
  const double inv_n = 1.0 / (double)n;
  for (int64_t j = threadIdx.x; j <= i; j += 256) {
    const int64_t pj = perm[d - 1 - j];
    const int64_t r = min(pi, pj), c = max(pi, pj);
    const double v = pi == pj ? (double)w.keys[pi] * inv_n + lam : (double)H[r * d + c] * inv_n;
    A[i * d + j] = (float)v;
  }
}

// ---------------------------------------------------------------- diagonal block: factor + inverse
//
// The 128 x 128 diagonal block is factored and inverted in LDS by one 256-thread workgroup, blocked
// by 16. One wave factors and inverts each 16 x 16 diagonal sub-block in registers (every value a
// lane needs from another lane arrives by a DPP row broadcast). Everything else is 16 x 16 MFMA
// tiles on the four waves, in two phases per sub-block step p:
//   A: the sub-panel solve L_qp = A_qp X_pp^T (q > p), and the finished blocks of row p of the
//      inverse, X_pj = -X_pp W_pj (j < p);
//   B: the symmetric update A_qr -= L_qp L_rp^T (p < r <= q) and the inverse's right-looking update
//      W_qj += L_qp X_pj (q > p, j <= p), where W_qj = sum_{t=j}^{q-1} L_qt X_tj accumulates in the
//      inverse's own tile (block forward substitution for L^-1, X_qj = -X_qq W_qj). Wave 0 instead
//      updates tile (p + 1, p + 1) and factors sub-block p + 1 while waves 1..3 do the rest.
constexpr int LDB = NB + 4;   // LDS leading dimension: 16 x 16 tiles read by rows or columns are conflict-free
constexpr int SB = 16;        // sub-block
constexpr int NS = NB / SB;   // sub-blocks per block
constexpr int LDT = SB + 1;   // per-wave temporary tile

// Register r of lane l of a 16 x 16 MFMA result holds row 4 (l / 16) + r, column l % 16.
GPTQ_DEV floatx4 tile_load(const float* T, int lane) {
  floatx4 v;
#pragma unroll
  for (int r = 0; r < 4; ++r) v[r] = T[(4 * (lane >> 4) + r) * LDB + (lane & 15)];
  return v;
}

GPTQ_DEV void tile_store(float* T, int lane, floatx4 v) {
#pragma unroll
  for (int r = 0; r < 4; ++r) T[(4 * (lane >> 4) + r) * LDB + (lane & 15)] = v[r];
}

// One tile product in LDS: C = (acc ? C : 0) + sgn * A op(B), with op(B) = B^T (bt) or B, all
// 16 x 16 tiles with leading dimension LDB (offsets in floats from the LDS base). C may be A or B
// (acc = 0 then): every read of a task precedes its store.
struct TileTask {
  int c, a, b, bt, acc;
  float sgn;
};

// v_mfma_f32_16x16x4f32 takes A[l % 16][k + l / 16] and B[k + l / 16][l % 16] from lane l. All of a
// task's operands are read before its first MFMA, so the LDS latency is paid once per task.
struct TileOps {
  float a[4], b[4];
  floatx4 c;
};

GPTQ_DEV TileOps tile_fetch(const float* sm, const TileTask& t, int lane) {
  TileOps o;
  const int r = lane & 15, kk = lane >> 4;
  const float* pa = sm + t.a + r * LDB + kk;
  const float* pb = sm + t.b + (t.bt ? r * LDB + kk : kk * LDB + r);
  const int sb = t.bt ? 4 : 4 * LDB;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    o.a[k] = pa[4 * k];
    o.b[k] = pb[k * sb];
  }
  o.c = t.acc ? tile_load(sm + t.c, lane) : floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  return o;
}

GPTQ_DEV floatx4 tile_mma(const TileOps& o, float sgn) {
  floatx4 acc = o.c;
#pragma unroll
  for (int k = 0; k < 4; ++k) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(sgn * o.a[k], o.b[k], acc, 0, 0, 0);
  return acc;
}

GPTQ_DEV void run_task(float* sm, const TileTask& t, int lane) {
  const TileOps o = tile_fetch(sm, t, lane);
  __builtin_amdgcn_sched_barrier(0);
  tile_store(sm + t.c, lane, tile_mma(o, t.sgn));
}

// Two independent tasks at once, so that the loads and MFMAs of both overlap.
GPTQ_DEV void run_task2(float* sm, const TileTask& t0, const TileTask& t1, int lane) {
  const TileOps o0 = tile_fetch(sm, t0, lane);
  const TileOps o1 = tile_fetch(sm, t1, lane);
  __builtin_amdgcn_sched_barrier(0);   // every read ahead of the first MFMA
  const floatx4 r0 = tile_mma(o0, t0.sgn);
  const floatx4 r1 = tile_mma(o1, t1.sgn);
  tile_store(sm + t0.c, lane, r0);
  tile_store(sm + t1.c, lane, r1);
}

// Runs the tasks a wave is given (a wave-uniform list) two at a time. No task of one phase reads a
// tile that another task of the phase writes.
struct TaskPair {
  float* sm;
  int lane, have;
  TileTask held;
  GPTQ_DEV void push(const TileTask& t) {
    if (have) {
      run_task2(sm, held, t, lane);
      have = 0;
    } else {
      held = t;
      have = 1;
    }
  }
  GPTQ_DEV void flush() {
    if (have) run_task(sm, held, lane);
    have = 0;
  }
};

// Column step J's updates of the 16 x 16 factor-and-inverse (see chol_inv16) as one block of DPP
// multiply-adds: a[c] -= (lane c's l) * l for c > J, and y[k] -= (lane J's y[k]) * m for the
// columns 4k + g that row J can reach (4k <= J). A DPP read needs two wait states after a VALU
// write of its source, which the compiler does not track through inline assembly: the leading s_nop
// covers the sources written before the block (none is written inside it), the trailing one covers
// a DPP read of the block's results right after it.
#define FA(c) "v_fmac_f32_dpp %[a" #c "], -%[l], %[l] row_newbcast:" #c " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
#define FY(k, j) "v_fmac_f32_dpp %[y" #k "], %[y" #k "], -%[m] row_newbcast:" #j " row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
#define CHOL16_OPERANDS                                                                                     \
  [a0] "+v"(a[0]), [a1] "+v"(a[1]), [a2] "+v"(a[2]), [a3] "+v"(a[3]), [a4] "+v"(a[4]), [a5] "+v"(a[5]),     \
      [a6] "+v"(a[6]), [a7] "+v"(a[7]), [a8] "+v"(a[8]), [a9] "+v"(a[9]), [a10] "+v"(a[10]),               \
      [a11] "+v"(a[11]), [a12] "+v"(a[12]), [a13] "+v"(a[13]), [a14] "+v"(a[14]), [a15] "+v"(a[15]),       \
      [y0] "+v"(y[0]), [y1] "+v"(y[1]), [y2] "+v"(y[2]), [y3] "+v"(y[3])                                  \
      : [l] "v"(l), [m] "v"(m)
template <int J>
GPTQ_DEV void chol16_step(float (&a)[SB], float (&y)[4], float l, float m) {
  if constexpr (J == 0) asm("s_nop 1\n\t" FA(1) FA(2) FA(3) FA(4) FA(5) FA(6) FA(7) FA(8) FA(9) FA(10) FA(11) FA(12) FA(13) FA(14) FA(15) FY(0, 0) "s_nop 1" : CHOL16_OPERANDS);
  if constexpr (J == 1) asm("s_nop 1\n\t" FA(2) FA(3) FA(4) FA(5) FA(6) FA(7) FA(8) FA(9) FA(10) FA(11) FA(12) FA(13) FA(14) FA(15) FY(0, 1) "s_nop 1" : CHOL16_OPERANDS);
  if constexpr (J == 2) asm("s_nop 1\n\t" FA(3) FA(4) FA(5) FA(6) FA(7) FA(8) FA(9) FA(10) FA(11) FA(12) FA(13) FA(14) FA(15) FY(0, 2) "s_nop 1" : CHOL16_OPERANDS);
  if constexpr (J == 3) asm("s_nop 1\n\t" FA(4) FA(5) FA(6) FA(7) FA(8) FA(9) FA(10) FA(11) FA(12) FA(13) FA(14) FA(15) FY(0, 3) "s_nop 1" : CHOL16_OPERANDS);
  if constexpr (J == 4) asm("s_nop 1\n\t" FA(5) FA(6) FA(7) FA(8) FA(9) FA(10) FA(11) FA(12) FA(13) FA(14) FA(15) FY(0, 4) FY(1, 4) "s_nop 1" : CHOL16_OPERANDS);
  if constexpr (J == 5) asm("s_nop 1\n\t" FA(6) FA(7) FA(8) FA(9) FA(10) FA(11) FA(12) FA(13) FA(14) FA(15) FY(0, 5) FY(1, 5) "s_nop 1" : CHOL16_OPERANDS);
  if constexpr (J == 6) asm("s_nop 1\n\t" FA(7) FA(8) FA(9) FA(10) FA(11) FA(12) FA(13) FA(14) FA(15) FY(0, 6) FY(1, 6) "s_nop 1" : CHOL16_OPERANDS);
  if constexpr (J == 7) asm("s_nop 1\n\t" FA(8) FA(9) FA(10) FA(11) FA(12) FA(13) FA(14) FA(15) FY(0, 7) FY(1, 7) "s_nop 1" : CHOL16_OPERANDS);
  if constexpr (J == 8) asm("s_nop 1\n\t" FA(9) FA(10) FA(11) FA(12) FA(13) FA(14) FA(15) FY(0, 8) FY(1, 8) FY(2, 8) "s_nop 1" : CHOL16_OPERANDS);
  if constexpr (J == 9) asm("s_nop 1\n\t" FA(10) FA(11) FA(12) FA(13) FA(14) FA(15) FY(0, 9) FY(1, 9) FY(2, 9) "s_nop 1" : CHOL16_OPERANDS);
  if constexpr (J == 10) asm("s_nop 1\n\t" FA(11) FA(12) FA(13) FA(14) FA(15) FY(0, 10) FY(1, 10) FY(2, 10) "s_nop 1" : CHOL16_OPERANDS);
  if constexpr (J == 11) asm("s_nop 1\n\t" FA(12) FA(13) FA(14) FA(15) FY(0, 11) FY(1, 11) FY(2, 11) "s_nop 1" : CHOL16_OPERANDS);
  if constexpr (J == 12) asm("s_nop 1\n\t" FA(13) FA(14) FA(15) FY(0, 12) FY(1, 12) FY(2, 12) FY(3, 12) "s_nop 1" : CHOL16_OPERANDS);
  if constexpr (J == 13) asm("s_nop 1\n\t" FA(14) FA(15) FY(0, 13) FY(1, 13) FY(2, 13) FY(3, 13) "s_nop 1" : CHOL16_OPERANDS);
  if constexpr (J == 14) asm("s_nop 1\n\t" FA(15) FY(0, 14) FY(1, 14) FY(2, 14) FY(3, 14) "s_nop 1" : CHOL16_OPERANDS);
  if constexpr (J == 15) asm("s_nop 1\n\t" FY(0, 15) FY(1, 15) FY(2, 15) FY(3, 15) "s_nop 1" : CHOL16_OPERANDS);
}
#undef FA
#undef FY
#undef CHOL16_OPERANDS

// One wave: Cholesky factor of the 16 x 16 lower block at S (in place) and its inverse into Xs.
// Lane l holds row i = l % 16 of the block in registers (the four 16-lane groups alike) and a
// quarter of row i of the inverse: group g = l / 16 holds columns 4k + g, k = 0..3. Column step j
// computes r_j = 1 / l_jj and column j of the factor; the same step is the j-th step of forward
// elimination for the inverse, kept with a unit diagonal (rows i > j subtract l_ij r_j times row j)
// and scaled by 1 / l_ii at the end, which gives the same rows as dividing row j by l_jj at its
// step. The pivot, column j of L and row j of the inverse reach the other lanes by DPP row
// broadcasts, and no step branches. Entries above the diagonal hold unread values and are zeroed on
// the way out. A pivot that is not positive gives l_jj <= 0 (or NaN); the first one is recorded in
// info (1-based index gbase + j + 1, when the column is real, j < valid), and the rest of the block
// is then unspecified.
GPTQ_DEV void chol_inv16(float* S, float* Xs, int lane, int64_t* info, int64_t gbase, int valid) {
  int ln = lane;
  asm("" : "+v"(ln));   // row tests derived per call, not hoisted out of the caller's loop
  const int i = ln & 15, g = ln >> 4;
  float a[SB], y[4], below[SB];
#pragma unroll
  for (int c = 0; c < SB; ++c) {
    const float v = S[i * LDB + c];
    a[c] = (c <= i) ? v : 0.0f;
    below[c] = (i > c) ? 1.0f : 0.0f;
    asm("" : "+v"(below[c]));   // used as a multiplier, not turned back into a select
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) y[k] = (4 * k + g == i) ? 1.0f : 0.0f;
  static_for<0, SB>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    const float p = row_bcast<j>(a[j]);
    const float r = fminf(__builtin_amdgcn_rsqf(p), FLT_MAX);   // 1 / l_jj (finite for any pivot)
    const float l = a[j] * r;                                    // l_ij
    const float m = l * r * below[j];                            // l_ij / l_jj for rows i > j, else 0
    a[j] = l;
    chol16_step<j>(a, y, l, m);
  });
  int ie = i;
  asm("" : "+v"(ie));   // fresh row tests for the stores (the load's would stay live throughout)
  if (lane < SB) {
#pragma unroll
    for (int c = 0; c < SB; ++c) S[ie * LDB + c] = (c <= ie) ? a[c] : 0.0f;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  const float lii = S[ie * LDB + ie];
  // first non-positive pivot (lanes 0..15 hold steps 0..15)
  const uint64_t badm = __builtin_amdgcn_ballot_w64(!(lii > 0.0f)) & 0xFFFFull;
  const int bad = badm ? __builtin_ctzll(badm) : SB;
  if (bad < SB && bad < valid && lane == 0 && *info == 0) *info = gbase + bad + 1;
  const float ri = __builtin_amdgcn_rcpf(lii);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int c = 4 * k + g;
    Xs[ie * LDB + c] = (c <= ie) ? y[k] * ri : 0.0f;
  }
}

GPTQ_DEV int tile_off(int base, int q, int r) { return base + (SB * q) * LDB + SB * r; }

// Block (q, pb) of the inverse, X_qp = -X_qq sum_{t=pb}^{q-1} L_qt X_tp, by one wave; T is the wave's
// 16 x 16 temporary (leading dimension LDT). The operands of two terms are read before their MFMAs.
GPTQ_DEV void inv_tile(float* sm, float* T, int q, int pb, int lane) {
  const int LA = 0, XA = NB * LDB;
  const int r = lane & 15, kk = lane >> 4;
  floatx4 acc = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  int t = pb;
  for (; t + 1 < q; t += 2) {
    const float* a0 = sm + tile_off(LA, q, t) + r * LDB + kk;
    const float* b0 = sm + tile_off(XA, t, pb) + kk * LDB + r;
    const float* a1 = a0 + SB;
    const float* b1 = sm + tile_off(XA, t + 1, pb) + kk * LDB + r;
    float av0[4], bv0[4], av1[4], bv1[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      av0[k] = a0[4 * k];
      bv0[k] = b0[4 * k * LDB];
      av1[k] = a1[4 * k];
      bv1[k] = b1[4 * k * LDB];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < 4; ++k) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av0[k], bv0[k], acc, 0, 0, 0);
#pragma unroll
    for (int k = 0; k < 4; ++k) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av1[k], bv1[k], acc, 0, 0, 0);
  }
  if (t < q) {
    const float* a0 = sm + tile_off(LA, q, t) + r * LDB + kk;
    const float* b0 = sm + tile_off(XA, t, pb) + kk * LDB + r;
    float av0[4], bv0[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      av0[k] = a0[4 * k];
      bv0[k] = b0[4 * k * LDB];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < 4; ++k) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av0[k], bv0[k], acc, 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) T[(4 * kk + i) * LDT + r] = acc[i];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  const float* xq = sm + tile_off(XA, q, q) + r * LDB + kk;
  float av[4], bv[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    av[k] = xq[4 * k];
    bv[k] = T[(4 * k + kk) * LDT + r];
  }
  __builtin_amdgcn_sched_barrier(0);
  acc = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int k = 0; k < 4; ++k) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(-av[k], bv[k], acc, 0, 0, 0);
  tile_store(sm + tile_off(XA, q, pb), lane, acc);
  __builtin_amdgcn_wave_barrier();   // T is reused by this wave's next tile
}

// Block row q of the inverse (blocks pb < q) on waves w = 0..nw-1: the chains are q - pb terms long,
// dealt longest first to the least-loaded wave (every wave computes the same deal).
GPTQ_DEV void inv_row(float* sm, float* T, int q, int w, int nw, int lane) {
  int load[4] = {0, 0, 0, 0};
  for (int pb = 0; pb < q; ++pb) {
    int best = 0;
    for (int u = 1; u < nw; ++u) best = load[u] < load[best] ? u : best;
    load[best] += q - pb + 1;
    if (best == w) inv_tile(sm, T, q, pb, lane);
  }
}

// Workgroup 0 factors the diagonal block at (k0, k0) (A = L L^T, lower) and replaces the whole block
// in A by the inverse of L (lower triangle; zeros above). A last block narrower than NB is padded with
// an identity, which leaves the factor and inverse of the real part unchanged. vec: A and d allow
// 16-byte row accesses. Workgroups 1.. copy `panel` (the column panel below the block, which the
// diagonal workgroup does not touch) to its staging buffer.
__global__ __launch_bounds__(256) void chol_diag_kernel(float* __restrict__ A, int64_t d, int64_t k0, int nb,
                                                        int vec, int64_t* __restrict__ info, Copy2D panel) {
  if (blockIdx.x > 0) {   // the other workgroups stage the column panel below the block
    copy_part(panel, blockIdx.x - 1, gridDim.x - 1);
    return;
  }
  extern __shared__ float sm[];
  float* La = sm;                 // [NB][LDB]: the block, then its Cholesky factor
  float* Xa = sm + NB * LDB;      // [NB][LDB]: the inverse of the factor
  float* Tt = sm + 2 * NB * LDB;  // [4][SB][LDT]: per-wave temporaries
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: task loops branch on scalars
  constexpr int PER = NB * NB / 256;
  constexpr int PER4 = PER / 4;
  if (nb == NB && vec) {
    float4 v[PER4];
#pragma unroll
    for (int q = 0; q < PER4; ++q) {
      const int e = tid + q * 256, r = e / (NB / 4), c = e % (NB / 4) * 4;
      v[q] = *reinterpret_cast<const float4*>(A + (k0 + r) * d + k0 + c);
    }
#pragma unroll
    for (int q = 0; q < PER4; ++q) {
      const int e = tid + q * 256, r = e / (NB / 4), c = e % (NB / 4) * 4;
      float4 x = v[q];
      x.x = (c <= r) ? x.x : 0.0f;
      x.y = (c + 1 <= r) ? x.y : 0.0f;
      x.z = (c + 2 <= r) ? x.z : 0.0f;
      x.w = (c + 3 <= r) ? x.w : 0.0f;
      *reinterpret_cast<float4*>(La + r * LDB + c) = x;
      *reinterpret_cast<float4*>(Xa + r * LDB + c) = float4{0.0f, 0.0f, 0.0f, 0.0f};
    }
  } else {
    for (int q = 0; q < PER; ++q) {
      const int e = tid + q * 256, r = e / NB, c = e % NB;
      float x = (r == c) ? 1.0f : 0.0f;
      if (r < nb && c <= r) x = A[(k0 + r) * d + k0 + c];
      La[r * LDB + c] = (c <= r) ? x : 0.0f;
      Xa[r * LDB + c] = 0.0f;
    }
  }
  __syncthreads();

  const int LA = 0, XA = NB * LDB;
  float* T = Tt + wave * SB * LDT;
  if (wave == 0) chol_inv16(La, Xa, lane, info, k0, nb);
  __syncthreads();
  for (int p = 0; p + 1 < NS; ++p) {
    {   // sub-panel solve: L_qp = A_qp X_pp^T for q > p
      TaskPair tp{sm, lane, 0, {}};
      for (int q = p + 1 + wave; q < NS; q += 4)
        tp.push(TileTask{tile_off(LA, q, p), tile_off(LA, q, p), tile_off(XA, p, p), 1, 0, 1.0f});
      tp.flush();
    }
    __syncthreads();
    // symmetric update A_qr -= L_qp L_rp^T for p < r <= q: tile (p + 1, p + 1) and the factor of
    // sub-block p + 1 on wave 0, the other tiles on waves 1..3
    if (wave == 0) {
      run_task(sm, TileTask{tile_off(LA, p + 1, p + 1), tile_off(LA, p + 1, p), tile_off(LA, p + 1, p), 1, 1, -1.0f},
               lane);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_wave_barrier();
      chol_inv16(La + (SB * (p + 1)) * LDB + SB * (p + 1), Xa + (SB * (p + 1)) * LDB + SB * (p + 1), lane, info,
                 k0 + SB * (p + 1), nb - SB * (p + 1));
    } else {
      TaskPair tp{sm, lane, 0, {}};
      int t = 0;
      for (int q = p + 2; q < NS; ++q)
        for (int r = p + 1; r <= q; ++r, ++t)
          if (t % 3 == wave - 1)
            tp.push(TileTask{tile_off(LA, q, r), tile_off(LA, q, p), tile_off(LA, r, p), 1, 1, -1.0f});
      tp.flush();
      // block row p of the inverse: its inputs (L_pt for t < p, X_pp, earlier rows) are final, and
      // nothing else in this phase touches it
      if (p > 0) inv_row(sm, T, p, wave - 1, 3, lane);
    }
    __syncthreads();
  }
  inv_row(sm, T, NS - 1, wave, 4, lane);   // the last block row of the inverse
  __syncthreads();
  if (nb == NB && vec) {
#pragma unroll
    for (int q = 0; q < PER4; ++q) {
      const int e = tid + q * 256, r = e / (NB / 4), c = e % (NB / 4) * 4;
      float4 x = *reinterpret_cast<const float4*>(Xa + r * LDB + c);
      x.x = (c <= r) ? x.x : 0.0f;
      x.y = (c + 1 <= r) ? x.y : 0.0f;
      x.z = (c + 2 <= r) ? x.z : 0.0f;
      x.w = (c + 3 <= r) ? x.w : 0.0f;
      *reinterpret_cast<float4*>(A + (k0 + r) * d + k0 + c) = x;
    }
  } else {
    for (int q = 0; q < PER; ++q) {
      const int e = tid + q * 256, r = e / NB, c = e % NB;
      if (r < nb && c < nb) A[(k0 + r) * d + k0 + c] = (c <= r) ? Xa[r * LDB + c] : 0.0f;
    }
  }
}

// 180-degree rotation in place: the lower triangle of the inverted reversed factor becomes U's
// upper triangle; U's strict lower triangle is set to zero.
__global__ __launch_bounds__(256) void flip_kernel(float* __restrict__ A, int64_t d) {
  const int64_t i = blockIdx.x;
  for (int64_t j = threadIdx.x; j < i; j += 256) {
    const float v = A[i * d + j];
    A[(d - 1 - i) * d + (d - 1 - j)] = v;
    A[i * d + j] = 0.0f;
  }
  if (threadIdx.x == 0 && i < d - 1 - i) {
    const float a = A[i * d + i], b = A[(d - 1 - i) * d + (d - 1 - i)];
    A[i * d + i] = b;
    A[(d - 1 - i) * d + (d - 1 - i)] = a;
  }
}

size_t chol_smem() { return ((size_t)2 * NB * LDB + 4 * SB * LDT) * sizeof(float); }

}  // namespace

// Workspace: the status words, the sort keys, and the panel buffers that stage the operand of the
// products that overwrite their own input: d x NB floats for the Cholesky's panel solve, and for the
// inverse d x NB for row panels and d x 2 NB for the two column panels of a pair of steps.
size_t factor_keys_bytes(int64_t d) { return ((size_t)d * sizeof(float) + 255) / 256 * 256; }
size_t factor_workspace_bytes(int64_t d) { return 256 + factor_keys_bytes(d) + 4 * (size_t)d * NB * sizeof(float); }

// Returns hipSuccess after queueing everything; *status_out / *info_out are device addresses of the
// status word and pivot index (read by the caller after a stream synchronisation).
hipError_t factor(const float* H, int64_t d, int64_t n, double damp, int act_order, float* U, int32_t* perm,
                  void* work, hipStream_t s, int** status_dev, int64_t** info_dev, bool one_stream) {
  char* wb = static_cast<char*>(work);
  FactorWork w;
  w.lam = reinterpret_cast<double*>(wb);
  w.info = reinterpret_cast<int64_t*>(wb + 8);
  w.status = reinterpret_cast<int*>(wb + 16);
  w.keys = reinterpret_cast<float*>(wb + 256);
  float* stage_main = reinterpret_cast<float*>(wb + 256 + factor_keys_bytes(d));   // d x NB, caller's stream
  float* stage_row = stage_main + d * NB;                                           // NB x d, helper stream
  float* stage_col = stage_row + d * NB;                                            // d x 2 NB, helper stream
  *status_dev = w.status;
  *info_dev = w.info;

  hipLaunchKernelGGL(diag_stats_kernel, dim3(1), dim3(1024), 0, s, H, d, n, damp, w);
  if (act_order)
    hipLaunchKernelGGL(rank_perm_kernel, dim3((unsigned)((d + 255) / 256)), dim3(256), 0, s, w.keys, d, perm);
  else
    hipLaunchKernelGGL(iota_kernel, dim3((unsigned)((d + 255) / 256)), dim3(256), 0, s, perm, d);
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)d), dim3(256), 0, s, H, d, n, perm, w, U);

  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute((const void*)chol_diag_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                        (int)chol_smem());
    attr = true;
  }
  // Blocked right-looking Cholesky of the reversed matrix on the caller's stream (diagonal blocks end
  // up inverted), and the blocked right-looking inverse of the factor on a helper stream hs. Inverse
  // step j starts after the group of Cholesky steps that holds step j is complete, its trailing
  // update included (that update reads the column panels the inverse steps overwrite), and touches
  // only columns left of block j + 1, which the later Cholesky steps neither read nor write. A cross-stream wait costs the host several
  // microseconds, so hs waits once per TB Cholesky steps (once per group of steps when the groups
  // below are longer) and then runs those inverse steps; with pairs the last TB steps go a pair at a
  // time, so that after the last Cholesky step only one pair of inverse steps is left. With
  // one_stream, hs is s itself and the steps simply follow one another.
  constexpr int64_t TB = 4;
  Helpers* hp = nullptr;
  hipError_t e = hipSuccess;
  hipStream_t hs = s;
  hipEvent_t ev_step = nullptr, ev_done = nullptr;
  if (!one_stream) {
    if ((e = helpers(&hp)) != hipSuccess) return e;
    hs = hp->stream[1];
    ev_step = hp->event[4];
    ev_done = hp->event[5];
    helpers_lock(hp);
  }
  const int64_t nblk = (d + NB - 1) / NB;
  const int vec = d % 4 == 0 && (uintptr_t)U % 16 == 0;
  // Cholesky step k on the caller's stream: the diagonal block (its kernel's other workgroups stage
  // the column panel P below it: the panel solve's workgroups of one row strip must not overwrite
  // the columns another one still reads), then the panel solve P <- P L_kk^-T
  auto chol_step = [&](int64_t k) -> hipError_t {
    const int64_t k0 = k * NB, k1 = std::min(d, k0 + NB), kb = k1 - k0;
    const Copy2D pc = make_copy(stage_main, kb, U + k1 * d + k0, d, d - k1, kb);
    hipLaunchKernelGGL(chol_diag_kernel, dim3(1 + copy_groups(d - k1, kb)), dim3(256), chol_smem(), s, U, d, k0,
                       (int)kb, vec, w.info, pc);
    hipError_t r = hipGetLastError();
    if (r != hipSuccess || k1 >= d) return r;
    GemmArgs t{};
    t.M = d - k1; t.N = kb; t.K = kb;
    t.A = stage_main; t.lda = kb; t.transA = 0;
    t.B = U + k0 * d + k0; t.ldb = d; t.transB = 1;
    t.C = U + k1 * d + k0; t.ldc = d;
    t.alpha = 1.0f; t.beta = 0.0f; t.tri = 0;
    return gemm_f32(t, s);
  };
  // Inverse step j on hs: with S_j = U[j0:j1, :j0] holding sum_t<j L_jt X_t, block row j of the
  // inverse is X_j = -X_jj S_j, and the rows below take their part of it, S_i += L_ij X_j, the block
  // column j of S_i being L_ij X_jj.
  auto inv_step = [&](int64_t k) -> hipError_t {
    const int64_t j0 = k * NB, j1 = std::min(d, j0 + NB), jb = j1 - j0;
    hipError_t st = hipSuccess;
    {
      // stage the row panel R = U[j0:j1, :j0] and the column panel L[j1:, j] together: nothing in
      // this step changes the column panel before its own product
      const Copy2D rc = make_copy(stage_row, j0, U + j0 * d, d, jb, j0);
      const Copy2D cc = make_copy(stage_col, jb, U + j1 * d + j0, d, d - j1, jb);
      const unsigned g0 = copy_groups(jb, j0), g1 = copy_groups(d - j1, jb);
      if (g0 + g1 > 0) {
        hipLaunchKernelGGL(copy2_kernel, dim3(g0 + g1), dim3(256), 0, hs, rc, cc, g0);
        if ((st = hipGetLastError()) != hipSuccess) return st;
      }
    }
    if (j0 > 0) {
      // row panel: R <- -X_jj R
      GemmArgs r{};
      r.M = jb; r.N = j0; r.K = jb;
      r.A = U + j0 * d + j0; r.lda = d; r.transA = 0;
      r.B = stage_row; r.ldb = j0; r.transB = 0;
      r.C = U + j0 * d; r.ldc = d;
      r.alpha = -1.0f; r.beta = 0.0f; r.tri = 0;
      if ((st = gemm_f32(r, hs)) != hipSuccess) return st;
      if (j1 < d) {
        GemmArgs q{};  // rectangle: A[j1:, :j0] += L[j1:, j] R
        q.M = d - j1; q.N = j0; q.K = jb;
        q.A = U + j1 * d + j0; q.lda = d; q.transA = 0;
        q.B = U + j0 * d; q.ldb = d; q.transB = 0;
        q.C = U + j1 * d; q.ldc = d;
        q.alpha = 1.0f; q.beta = 1.0f; q.tri = 0;
        if ((st = gemm_f32(q, hs)) != hipSuccess) return st;
      }
    }
    if (j1 < d) {
      // column panel: L[j1:, j] <- L[j1:, j] X_jj
      GemmArgs c{};
      c.M = d - j1; c.N = jb; c.K = jb;
      c.A = stage_col; c.lda = jb; c.transA = 0;
      c.B = U + j0 * d + j0; c.ldb = d; c.transB = 0;
      c.C = U + j1 * d + j0; c.ldc = d;
      c.alpha = 1.0f; c.beta = 0.0f; c.tri = 0;
      if ((st = gemm_f32(c, hs)) != hipSuccess) return st;
    }
    return hipSuccess;
  };
  // Inverse steps j and j + 1 together: row j, then row block j + 1's part of it (S_j+1 += L_j+1,j X_j
  // and its block column j, L_j+1,j X_jj), row j + 1, and then the rows below j2 take both rows' parts
  // in products with K = 2 NB: S_i[:, :j0] += [L_ij L_i,j+1] [X_j; X_j+1] and block column j of S_i
  // = [L_ij L_i,j+1] [X_jj; X_j+1,j]; block column j + 1 is L_i,j+1 X_j+1,j+1. The column panels
  // L[j1:, j0:j2] are staged first, since the products overwrite them.
  auto inv_pair = [&](int64_t k) -> hipError_t {
    const int64_t j0 = k * NB, j1 = j0 + NB, j2 = std::min(d, j1 + NB);
    const int64_t jb = NB, jb2 = j2 - j1, w2 = j2 - j0;
    hipError_t r = hipSuccess;
    auto gemm = [&](int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, const float* B, int64_t ldb,
                    float* C, float alpha, float beta) {
      GemmArgs g{};
      g.M = M; g.N = N; g.K = K;
      g.A = A; g.lda = lda; g.transA = 0;
      g.B = B; g.ldb = ldb; g.transB = 0;
      g.C = C; g.ldc = d;
      g.alpha = alpha; g.beta = beta; g.tri = 0;
      return gemm_f32(g, hs);
    };
    {
      const Copy2D rc = make_copy(stage_row, j0, U + j0 * d, d, jb, j0);
      const Copy2D cc = make_copy(stage_col, w2, U + j1 * d + j0, d, d - j1, w2);
      const unsigned g0 = copy_groups(jb, j0), g1 = copy_groups(d - j1, w2);
      hipLaunchKernelGGL(copy2_kernel, dim3(g0 + g1), dim3(256), 0, hs, rc, cc, g0);
      if ((r = hipGetLastError()) != hipSuccess) return r;
    }
    if (j0 > 0) {
      if ((r = gemm(jb, j0, jb, U + j0 * d + j0, d, stage_row, j0, U + j0 * d, -1.0f, 0.0f)) != hipSuccess) return r;
      if ((r = gemm(jb2, j0, jb, stage_col, w2, U + j0 * d, d, U + j1 * d, 1.0f, 1.0f)) != hipSuccess) return r;
    }
    if ((r = gemm(jb2, jb, jb, stage_col, w2, U + j0 * d + j0, d, U + j1 * d + j0, 1.0f, 0.0f)) != hipSuccess) return r;
    {
      const Copy2D rc = make_copy(stage_row, j1, U + j1 * d, d, jb2, j1);
      const Copy2D none = make_copy(stage_row, j1, U + j1 * d, d, 0, 0);
      hipLaunchKernelGGL(copy2_kernel, dim3(copy_groups(jb2, j1)), dim3(256), 0, hs, rc, none, copy_groups(jb2, j1));
      if ((r = hipGetLastError()) != hipSuccess) return r;
    }
    if ((r = gemm(jb2, j1, jb2, U + j1 * d + j1, d, stage_row, j1, U + j1 * d, -1.0f, 0.0f)) != hipSuccess) return r;
    if (j2 < d) {
      const float* Lb = stage_col + jb2 * w2;   // rows j2.. of the staged column panels
      if (j0 > 0 && (r = gemm(d - j2, j0, w2, Lb, w2, U + j0 * d, d, U + j2 * d, 1.0f, 1.0f)) != hipSuccess) return r;
      if ((r = gemm(d - j2, jb, w2, Lb, w2, U + j0 * d + j0, d, U + j2 * d + j0, 1.0f, 0.0f)) != hipSuccess) return r;
      if ((r = gemm(d - j2, jb2, jb2, Lb + jb, w2, U + j1 * d + j1, d, U + j2 * d + j1, 1.0f, 0.0f)) != hipSuccess)
        return r;
    }
    return hipSuccess;
  };
  // The trailing updates go by groups of G adjacent steps. After each panel solve of a group only the
  // group's later block columns take its update, A[k1:, k1:ge] -= P_k P_k[0:ge-k1]^T (their diagonal
  // blocks whole: the part above the diagonal is never read and the diagonal kernel rewrites it);
  // after the group's last step the rest takes all of the group's panels in one product,
  // A[ge:, ge:] -= P P^T (lower part, K = G NB: the panels are adjacent columns of A).
  // G: 2 below d = 8192, 4 up to 32768, 8 beyond (measured: d = 49152 786 ms with pairs, 740 with
  // groups of 4, 721 with 8; d = 11008 13.6, 13.4 and 13.5 ms; d = 4096 keeps pairs, whose
  // diagonal blocks set its pace)
  const int64_t G = d >= 32768 ? 8 : d >= 8192 ? 4 : 2;
  for (int64_t kt = 0, kend = 0; kt < nblk && e == hipSuccess; kt = kend) {
    // batches of TB steps that end on group boundaries, the last ones a group at a time
    kend = G > 2 ? std::min(nblk, kt + G) : std::min(nblk, kt + TB <= nblk - TB ? kt + TB : kt + 2);
    for (int64_t g0 = kt; g0 < kend && e == hipSuccess; g0 += G) {
      const int64_t gend = std::min(kend, g0 + G), ge = std::min(d, gend * NB);
      for (int64_t k = g0; k < gend && e == hipSuccess; ++k) {
        const int64_t k0 = k * NB, k1 = std::min(d, k0 + NB), kb = k1 - k0;
        if ((e = chol_step(k)) != hipSuccess) break;
        if (k1 >= ge) break;
        GemmArgs ua{};
        ua.M = d - k1; ua.N = ge - k1; ua.K = kb;
        ua.A = U + k1 * d + k0; ua.lda = d; ua.transA = 0;
        ua.B = U + k1 * d + k0; ua.ldb = d; ua.transB = 1;
        ua.C = U + k1 * d + k1; ua.ldc = d;
        ua.alpha = -1.0f; ua.beta = 1.0f; ua.tri = 0;
        e = gemm_f32(ua, s);
      }
      if (e == hipSuccess && ge < d) {
        GemmArgs ub{};
        ub.M = d - ge; ub.N = d - ge; ub.K = ge - g0 * NB;
        ub.A = U + ge * d + g0 * NB; ub.lda = d; ub.transA = 0;
        ub.B = U + ge * d + g0 * NB; ub.ldb = d; ub.transB = 1;
        ub.C = U + ge * d + ge; ub.ldc = d;
        ub.alpha = -1.0f; ub.beta = 1.0f; ub.tri = 1;
        e = gemm_f32(ub, s);
      }
    }
    if (e != hipSuccess) break;
    if (!one_stream) {
      if ((e = hipEventRecord(ev_step, s)) != hipSuccess) break;
      if ((e = hipStreamWaitEvent(hs, ev_step, 0)) != hipSuccess) break;
    }
    // inverse steps kt .. kend - 1 on hs (their diagonal blocks are already inverted), a pair at a
    // time where the products are large enough for K = 2 NB to pay (measured: 3 % faster at
    // d = 11008, 9 % at d = 49152, 2 % slower at d = 4096); the same steps with one_stream, so that
    // both give the same U bit for bit
    for (int64_t k = kt; k < kend && e == hipSuccess;) {
      if (d >= 8192 && k + 1 < kend) {
        e = inv_pair(k);
        k += 2;
      } else {
        e = inv_step(k);
        k += 1;
      }
    }
  }
  if (!one_stream) {
    // join the helper stream (also after a failed launch, so nothing is left behind)
    hipError_t j = hipEventRecord(ev_done, hs);
    if (j == hipSuccess) j = hipStreamWaitEvent(s, ev_done, 0);
    helpers_unlock(hp);
    if (e == hipSuccess) e = j;
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(flip_kernel, dim3((unsigned)d), dim3(256), 0, s, U, d);
  return hipGetLastError();
}

}  // namespace gptq
