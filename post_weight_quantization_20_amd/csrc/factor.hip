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

// dst[r][c] = src[r][c] for a rows x cols block (leading dimensions ldd, lds); used to stage the
// operand of a product whose output overwrites it. One thread per 4 consecutive elements of a row,
// moved as one 16-byte access when both sides allow it.
__global__ __launch_bounds__(256) void copy2d_kernel(float* __restrict__ dst, int64_t ldd, const float* __restrict__ src,
                                                     int64_t lds, int64_t rows, int64_t cols, int vec) {
  const int64_t c4 = (cols + 3) / 4, total = rows * c4;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / c4, c = (i % c4) * 4;
    if (vec && c + 4 <= cols) {
      *reinterpret_cast<float4*>(dst + r * ldd + c) = *reinterpret_cast<const float4*>(src + r * lds + c);
    } else {
      for (int64_t e = c; e < cols && e < c + 4; ++e) dst[r * ldd + e] = src[r * lds + e];
    }
  }
}

hipError_t copy2d(float* dst, int64_t ldd, const float* src, int64_t lds, int64_t rows, int64_t cols, hipStream_t s) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  const int vec = (uintptr_t)dst % 16 == 0 && (uintptr_t)src % 16 == 0 && ldd % 4 == 0 && lds % 4 == 0;
  const int64_t work = rows * ((cols + 3) / 4);
  const unsigned grid = (unsigned)std::min<int64_t>((work + 255) / 256, 4096);
  hipLaunchKernelGGL(copy2d_kernel, dim3(grid), dim3(256), 0, s, dst, ldd, src, lds, rows, cols, vec);
  return hipGetLastError();
}

__global__ void iota_kernel(int32_t* perm, int64_t d) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < d) perm[i] = (int32_t)i;
}

// A[i][j] (j <= i) = Hhat[p(i)][p(j)], p(i) = perm[d-1-i]: the damped, normalised Hessian in
// processing order, reversed. H's upper triangle is authoritative.
__global__ __launch_bounds__(256) void gather_kernel(const float* __restrict__ H, int64_t d, int64_t n,
                                                     const int32_t* __restrict__ perm, FactorWork w,
                                                     float* __restrict__ A) {
  const int64_t i = blockIdx.x;
  const int64_t pi = perm[d - 1 - i];
  const double lam = *w.lam;
  const double inv_n = 1.0 / (double)n;
  for (int64_t j = threadIdx.x; j <= i; j += 256) {
    const int64_t pj = perm[d - 1 - j];
    const int64_t r = min(pi, pj), c = max(pi, pj);
    double v = (double)H[r * d + c] * inv_n;
    if (pi == pj) v += lam;
    A[i * d + j] = (float)v;
  }
}

// ---------------------------------------------------------------- diagonal block: factor + inverse
//
// The 128 x 128 diagonal block is factored and inverted in LDS by one 256-thread workgroup, blocked
// by 16: for each 16-column sub-panel, one wave factors and inverts the 16 x 16 diagonal sub-block
// in registers (lane i holds row i; every value a lane needs from another lane arrives by a DPP
// row broadcast, so a column step costs a few VALU latencies), then the four waves apply the
// sub-panel solve and the symmetric update to the rest of the block as 16 x 16 MFMA tiles. The
// off-diagonal blocks of the inverse follow from block forward substitution,
// X_qp = -X_qq sum_{t=p}^{q-1} L_qt X_tp, again as MFMA tiles.
constexpr int LDB = NB + 4;   // LDS leading dimension: 16 x 16 tiles read by rows or columns are conflict-free
constexpr int SB = 16;        // sub-block
constexpr int LDT = SB + 1;   // per-wave temporary tile

// acc (+)= sa op(A) op(B) over K (a multiple of 4) for one 16 x 16 tile; A, B in LDS. op(A): A[i][k]
// or (TA) A[k][i]; op(B): B[k][j] or (TB) B[j][k]. One wave: v_mfma_f32_16x16x4f32 takes
// A[l % 16][k + l / 16] and B[k + l / 16][l % 16] from lane l.
template <bool TA, bool TB>
GPTQ_DEV floatx4 mma16(floatx4 acc, const float* A, int lda, const float* B, int ldb, int K, int lane,
                       float sa = 1.0f) {
  const int r = lane & 15, kk = lane >> 4;
  for (int k = 0; k < K; k += 4) {
    const float av = TA ? A[(k + kk) * lda + r] : A[r * lda + k + kk];
    const float bv = TB ? B[r * ldb + k + kk] : B[(k + kk) * ldb + r];
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(sa * av, bv, acc, 0, 0, 0);
  }
  return acc;
}

// Register r of lane l of a 16 x 16 MFMA result holds row 4 (l / 16) + r, column l % 16.
GPTQ_DEV floatx4 tile_load(const float* T, int ld, int lane) {
  floatx4 v;
#pragma unroll
  for (int r = 0; r < 4; ++r) v[r] = T[(4 * (lane >> 4) + r) * ld + (lane & 15)];
  return v;
}

GPTQ_DEV void tile_store(float* T, int ld, int lane, floatx4 v, float scale = 1.0f) {
#pragma unroll
  for (int r = 0; r < 4; ++r) T[(4 * (lane >> 4) + r) * ld + (lane & 15)] = scale * v[r];
}

GPTQ_DEV floatx4 zero4() { return floatx4{0.0f, 0.0f, 0.0f, 0.0f}; }

// One wave: Cholesky factor of the 16 x 16 lower block at S (in place) and its inverse into Xs.
// Lane i holds row i of the block and row i of the inverse in registers (each 16-lane row of the
// wave computes the same thing). Column step j computes l_jj and column j of the factor; the same
// step is the j-th step of forward elimination for the inverse (row j of L^-1 is final once divided
// by l_jj, then rows i > j subtract l_ij times it). The pivot, column j of L and row j of L^-1
// reach the other lanes by DPP row broadcasts, and no step branches. Entries above the diagonal
// are never read and are zeroed on the way out. A non-positive pivot is recorded in info (1-based
// index gbase + j + 1, when the column is real, j < valid) and replaced by 1.
GPTQ_DEV void chol_inv16(float* S, float* Xs, int lane, int64_t* info, int64_t gbase, int valid) {
  const int i = lane & 15;
  float a[SB], x[SB];
#pragma unroll
  for (int c = 0; c < SB; ++c) {
    a[c] = (c <= i) ? S[i * LDB + c] : 0.0f;
    x[c] = (c == i) ? 1.0f : 0.0f;
  }
  int bad = SB;   // first non-positive pivot
  static_for<0, SB>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    float p = row_bcast<j>(a[j]);
    const bool ok = p > 0.0f;
    bad = (!ok && j < bad) ? j : bad;
    p = ok ? p : 1.0f;
    const float r = __builtin_amdgcn_rsqf(p);   // 1 / l_jj
    const float lij = a[j] * r;                 // l_ij for rows i > j
    const float sx = (i == j) ? r : 1.0f;
#pragma unroll
    for (int c = 0; c <= j; ++c) x[c] *= sx;
    a[j] = (i > j) ? lij : ((i == j) ? p * r : 0.0f);
    static_for<j + 1, SB>([&](auto cc) {
      constexpr int c = decltype(cc)::value;
      a[c] = __builtin_fmaf(-lij, row_bcast<c>(lij), a[c]);
    });
    const float lx = (i > j) ? lij : 0.0f;
    static_for<0, j + 1>([&](auto cc) {
      constexpr int c = decltype(cc)::value;
      x[c] = __builtin_fmaf(-lx, row_bcast<j>(x[c]), x[c]);
    });
  });
  if (bad < SB && bad < valid && lane == 0 && *info == 0) *info = gbase + bad + 1;
  if (lane < SB) {
#pragma unroll
    for (int c = 0; c < SB; ++c) {
      S[i * LDB + c] = (c <= i) ? a[c] : 0.0f;
      Xs[i * LDB + c] = (c <= i) ? x[c] : 0.0f;
    }
  }
}

// Factors the diagonal block at (k0, k0) (A = L L^T, lower) and replaces the whole block in A by the
// inverse of L (lower triangle; zeros above). A last block narrower than NB is padded with an
// identity, which leaves the factor and inverse of the real part unchanged.
__global__ __launch_bounds__(256) void chol_diag_kernel(float* __restrict__ A, int64_t d, int64_t k0, int nb,
                                                        int64_t* __restrict__ info) {
  extern __shared__ float sm[];
  float* La = sm;                 // [NB][LDB]: the block, then its Cholesky factor
  float* Xa = sm + NB * LDB;      // [NB][LDB]: the inverse of the factor
  float* Tt = sm + 2 * NB * LDB;  // [4][SB][LDT]: per-wave temporaries
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int PER = NB * NB / 256;
  if (nb == NB) {
    float v[PER];
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int e = tid + q * 256, r = e / NB, c = e % NB;
      v[q] = A[(k0 + r) * d + k0 + c];
    }
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int e = tid + q * 256, r = e / NB, c = e % NB;
      La[r * LDB + c] = (c <= r) ? v[q] : 0.0f;
      Xa[r * LDB + c] = 0.0f;
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

  constexpr int NS = NB / SB;
  for (int p = 0; p < NS; ++p) {
    float* Dpp = La + (SB * p) * LDB + SB * p;
    float* Xpp = Xa + (SB * p) * LDB + SB * p;
    if (wave == 0) chol_inv16(Dpp, Xpp, lane, info, k0 + SB * p, nb - SB * p);
    __syncthreads();
    // sub-panel solve: L_qp = A_qp X_pp^T for q > p
    for (int q = p + 1 + wave; q < NS; q += 4) {
      float* Aqp = La + (SB * q) * LDB + SB * p;
      tile_store(Aqp, LDB, lane, mma16<false, true>(zero4(), Aqp, LDB, Xpp, LDB, SB, lane));
    }
    __syncthreads();
    // symmetric update: A_qr -= L_qp L_rp^T for p < r <= q
    {
      int t = 0;
      for (int q = p + 1; q < NS; ++q)
        for (int r = p + 1; r <= q; ++r, ++t) {
          if (t % 4 != wave) continue;
          float* Aqr = La + (SB * q) * LDB + SB * r;
          floatx4 acc = tile_load(Aqr, LDB, lane);
          acc = mma16<false, true>(acc, La + (SB * q) * LDB + SB * p, LDB, La + (SB * r) * LDB + SB * p, LDB, SB,
                                   lane, -1.0f);
          tile_store(Aqr, LDB, lane, acc);
        }
    }
    __syncthreads();
  }
  // off-diagonal blocks of the inverse, block row by block row
  for (int q = 1; q < NS; ++q) {
    for (int pb = wave; pb < q; pb += 4) {
      floatx4 acc = zero4();
      for (int t = pb; t < q; ++t)
        acc = mma16<false, false>(acc, La + (SB * q) * LDB + SB * t, LDB, Xa + (SB * t) * LDB + SB * pb, LDB, SB,
                                  lane);
      float* T = Tt + wave * SB * LDT;
      tile_store(T, LDT, lane, acc);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_wave_barrier();
      acc = mma16<false, false>(zero4(), Xa + (SB * q) * LDB + SB * q, LDB, T, LDT, SB, lane);
      tile_store(Xa + (SB * q) * LDB + SB * pb, LDB, lane, acc, -1.0f);
      __builtin_amdgcn_wave_barrier();
    }
    __syncthreads();
  }
  if (nb == NB) {
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int e = tid + q * 256, r = e / NB, c = e % NB;
      A[(k0 + r) * d + k0 + c] = (c <= r) ? Xa[r * LDB + c] : 0.0f;
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

// Workspace: the status words, the sort keys, and two panel buffers of d x NB floats (one per stream)
// that stage the operand of the three products that overwrite their own input.
size_t factor_keys_bytes(int64_t d) { return ((size_t)d * sizeof(float) + 255) / 256 * 256; }
size_t factor_workspace_bytes(int64_t d) { return 256 + factor_keys_bytes(d) + 2 * (size_t)d * NB * sizeof(float); }

// Returns hipSuccess after queueing everything; *status_out / *info_out are device addresses of the
// status word and pivot index (read by the caller after a stream synchronisation).
hipError_t factor(const float* H, int64_t d, int64_t n, double damp, int act_order, float* U, int32_t* perm,
                  void* work, hipStream_t s, int** status_dev, int64_t** info_dev) {
  char* wb = static_cast<char*>(work);
  FactorWork w;
  w.lam = reinterpret_cast<double*>(wb);
  w.info = reinterpret_cast<int64_t*>(wb + 8);
  w.status = reinterpret_cast<int*>(wb + 16);
  w.keys = reinterpret_cast<float*>(wb + 256);
  float* stage_main = reinterpret_cast<float*>(wb + 256 + factor_keys_bytes(d));   // d x NB, caller's stream
  float* stage_help = stage_main + d * NB;                                          // d x NB, helper stream
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
  // up inverted), and the blocked right-looking inverse of the factor on a helper stream. Inverse
  // step j starts after Cholesky step j is complete, its trailing update included (that update reads
  // the column panel the inverse step overwrites), and touches only columns left of block j + 1,
  // which the later Cholesky steps neither read nor write.
  Helpers* hp = nullptr;
  hipError_t e = helpers(&hp);
  if (e != hipSuccess) return e;
  hipStream_t hs = hp->stream[1];
  hipEvent_t ev_step = hp->event[4], ev_done = hp->event[5];
  helpers_lock(hp);
  const int64_t nblk = (d + NB - 1) / NB;
  for (int64_t k = 0; k < nblk && e == hipSuccess; ++k) {
    const int64_t k0 = k * NB, k1 = std::min(d, k0 + NB), kb = k1 - k0;
    hipLaunchKernelGGL(chol_diag_kernel, dim3(1), dim3(256), chol_smem(), s, U, d, k0, (int)kb, w.info);
    if (k1 < d) {
      // panel solve: P <- P L_kk^-T (P staged: workgroups of one row strip must not overwrite the
      // columns another one still reads)
      if ((e = copy2d(stage_main, kb, U + k1 * d + k0, d, d - k1, kb, s)) != hipSuccess) break;
      GemmArgs t{};
      t.M = d - k1; t.N = kb; t.K = kb;
      t.A = stage_main; t.lda = kb; t.transA = 0;
      t.B = U + k0 * d + k0; t.ldb = d; t.transB = 1;
      t.C = U + k1 * d + k0; t.ldc = d;
      t.alpha = 1.0f; t.beta = 0.0f; t.tri = 0;
      if ((e = gemm_f32(t, s)) != hipSuccess) break;
    }
    if (k1 < d) {
      GemmArgs u{};  // trailing update: A22 -= P P^T (lower part)
      u.M = d - k1; u.N = d - k1; u.K = kb;
      u.A = U + k1 * d + k0; u.lda = d; u.transA = 0;
      u.B = U + k1 * d + k0; u.ldb = d; u.transB = 1;
      u.C = U + k1 * d + k1; u.ldc = d;
      u.alpha = -1.0f; u.beta = 1.0f; u.tri = 1;
      if ((e = gemm_f32(u, s)) != hipSuccess) break;
    }
    if ((e = hipEventRecord(ev_step, s)) != hipSuccess) break;
    // inverse step k on the helper stream (the diagonal block is already inverted)
    if ((e = hipStreamWaitEvent(hs, ev_step, 0)) != hipSuccess) break;
    const int64_t j0 = k0, j1 = k1, jb = kb;
    if (j0 > 0) {
      // row panel: R <- -X_jj R (R staged)
      if ((e = copy2d(stage_help, j0, U + j0 * d, d, jb, j0, hs)) != hipSuccess) break;
      GemmArgs r{};
      r.M = jb; r.N = j0; r.K = jb;
      r.A = U + j0 * d + j0; r.lda = d; r.transA = 0;
      r.B = stage_help; r.ldb = j0; r.transB = 0;
      r.C = U + j0 * d; r.ldc = d;
      r.alpha = -1.0f; r.beta = 0.0f; r.tri = 0;
      if ((e = gemm_f32(r, hs)) != hipSuccess) break;
      if (j1 < d) {
        GemmArgs q{};  // rectangle: A[j1:, :j0] += L[j1:, j] R
        q.M = d - j1; q.N = j0; q.K = jb;
        q.A = U + j1 * d + j0; q.lda = d; q.transA = 0;
        q.B = U + j0 * d; q.ldb = d; q.transB = 0;
        q.C = U + j1 * d; q.ldc = d;
        q.alpha = 1.0f; q.beta = 1.0f; q.tri = 0;
        if ((e = gemm_f32(q, hs)) != hipSuccess) break;
      }
    }
    if (j1 < d) {
      // column panel: L[j1:, j] <- L[j1:, j] X_jj (L[j1:, j] staged)
      if ((e = copy2d(stage_help, jb, U + j1 * d + j0, d, d - j1, jb, hs)) != hipSuccess) break;
      GemmArgs c{};
      c.M = d - j1; c.N = jb; c.K = jb;
      c.A = stage_help; c.lda = jb; c.transA = 0;
      c.B = U + j0 * d + j0; c.ldb = d; c.transB = 0;
      c.C = U + j1 * d + j0; c.ldc = d;
      c.alpha = 1.0f; c.beta = 0.0f; c.tri = 0;
      if ((e = gemm_f32(c, hs)) != hipSuccess) break;
    }
  }
  // join the helper stream (also after a failed launch, so nothing is left behind)
  hipError_t j = hipEventRecord(ev_done, hs);
  if (j == hipSuccess) j = hipStreamWaitEvent(s, ev_done, 0);
  helpers_unlock(hp);
  if (e == hipSuccess) e = j;
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(flip_kernel, dim3((unsigned)d), dim3(256), 0, s, U, d);
  return hipGetLastError();
}

}  // namespace gptq
