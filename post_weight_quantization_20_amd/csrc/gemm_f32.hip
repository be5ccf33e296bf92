// fp32 GEMM on CDNA4 matrix cores (v_mfma_f32_32x32x2_f32).
//
// Used for every dense fp32 product of the solver: the lazy-batch trailing update of the column
// loop (GPTQ tools page, "How it works", Step 7), the panel solves, symmetric rank-k updates and
// triangular-inverse products of the factor (Step 6), and the Hessian of fp32 activations (Step 3).
//
// Tiling: a 256-thread workgroup (4 wave64s in a 2x2 grid) owns a 128x128 tile of C; each wave
// owns 64x64 = 2x2 MFMA blocks of 32x32 held in 64 accumulator registers per lane. The reduction
// dimension is staged through LDS 16 at a time, k-major (As[k][m], Bs[k][n]), double buffered,
// with the next stage's global loads in flight while the current stage feeds the MFMAs.
#include "common.hpp"

namespace gptq {
namespace {

constexpr int GT = 128;   // tile rows / cols
constexpr int GK = 16;    // k per LDS stage
constexpr int GP = 4;     // LDS row padding (floats)

// One operand tile stage: logical element (k, r) for k in [0, GK), r in [0, GT).
// KCONTIG: the stored matrix has k contiguous (element at P[r * ld + k]); otherwise r is
// contiguous (element at P[k * ld + r]). Each of the 256 threads moves two float4.
template <bool KCONTIG>
struct TileLoader {
  float4 v[2];

  GPTQ_DEV void load(const float* __restrict__ P, int64_t ld, int64_t r0, int64_t R, int64_t k0, int64_t K,
                     bool vec, int tid) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      int idx = tid + i * 256;
      int64_t r, k;
      if (KCONTIG) { r = r0 + (idx >> 2); k = k0 + ((idx & 3) << 2); }
      else         { k = k0 + (idx >> 5); r = r0 + ((idx & 31) << 2); }
      float t[4];
      if (KCONTIG) {
        const float* p = P + r * ld + k;
        if (vec && r < R && k + 3 < K) {
          float4 q = *reinterpret_cast<const float4*>(p);
          t[0] = q.x; t[1] = q.y; t[2] = q.z; t[3] = q.w;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) t[e] = (r < R && k + e < K) ? p[e] : 0.0f;
        }
      } else {
        const float* p = P + k * ld + r;
        if (vec && k < K && r + 3 < R) {
          float4 q = *reinterpret_cast<const float4*>(p);
          t[0] = q.x; t[1] = q.y; t[2] = q.z; t[3] = q.w;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) t[e] = (k < K && r + e < R) ? p[e] : 0.0f;
        }
      }
      v[i] = make_float4(t[0], t[1], t[2], t[3]);
    }
  }

  GPTQ_DEV void store(float (*S)[GT + GP], int tid) const {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      int idx = tid + i * 256;
      if (KCONTIG) {
        int r = idx >> 2, k = (idx & 3) << 2;
        S[k + 0][r] = v[i].x; S[k + 1][r] = v[i].y; S[k + 2][r] = v[i].z; S[k + 3][r] = v[i].w;
      } else {
        int k = idx >> 5, r = (idx & 31) << 2;
        *reinterpret_cast<float4*>(&S[k][r]) = v[i];
      }
    }
  }
};

template <bool AK, bool BK>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs a, int64_t tiles_n, int vecA, int vecB) {
  const int64_t tile = blockIdx.x;
  const int64_t tm = tile / tiles_n, tn = tile % tiles_n;
  const int64_t m0 = tm * GT, n0 = tn * GT;
  if (a.tri == 1 && m0 + GT - 1 < n0) return;
  if (a.tri == 2 && n0 + GT - 1 < m0) return;

  __shared__ float As[2][GK][GT + GP];
  __shared__ float Bs[2][GK][GT + GP];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int li = lane & 31, lk = lane >> 5;

  floatx16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  TileLoader<AK> la;  // op(A) tile: rows m, reduction k
  TileLoader<BK> lb;  // op(B) tile: cols n, reduction k
  const int64_t nk = (a.K + GK - 1) / GK;

  if (nk > 0) {
    la.load(a.A, a.lda, m0, a.M, 0, a.K, vecA, tid);
    lb.load(a.B, a.ldb, n0, a.N, 0, a.K, vecB, tid);
    la.store(As[0], tid);
    lb.store(Bs[0], tid);
  }
  __syncthreads();

  for (int64_t kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      la.load(a.A, a.lda, m0, a.M, (kt + 1) * GK, a.K, vecA, tid);
      lb.load(a.B, a.ldb, n0, a.N, (kt + 1) * GK, a.K, vecB, tid);
    }
#pragma unroll
    for (int ks = 0; ks < GK; ks += 2) {
      float av[2], bv[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) av[i] = As[cur][ks + lk][wm * 64 + i * 32 + li];
#pragma unroll
      for (int j = 0; j < 2; ++j) bv[j] = Bs[cur][ks + lk][wn * 64 + j * 32 + li];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[i], bv[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      la.store(As[cur ^ 1], tid);
      lb.store(Bs[cur ^ 1], tid);
    }
    __syncthreads();
  }

  // Epilogue. Accumulator register r of lane l holds row 8*(r/4) + 4*(l/32) + r%4, column l%32
  // of its 32x32 block.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * lk + (r & 3);
        const int64_t n = n0 + wn * 64 + j * 32 + li;
        if (m >= a.M || n >= a.N) continue;
        if (a.tri == 1 && m < n) continue;
        if (a.tri == 2 && m > n) continue;
        float* c = a.C + m * a.ldc + n;
        float v = a.alpha * acc[i][j][r];
        if (a.beta != 0.0f) v = __builtin_fmaf(a.beta, *c, v);
        *c = v;
      }
}

bool aligned16(const void* p, int64_t ld) { return ((uintptr_t)p % 16 == 0) && (ld % 4 == 0); }

}  // namespace

hipError_t gemm_f32(const GemmArgs& a, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  const int64_t tiles_m = (a.M + GT - 1) / GT, tiles_n = (a.N + GT - 1) / GT;
  const dim3 grid((unsigned)(tiles_m * tiles_n));
  // op(A) has k contiguous when A is not transposed; op(B) has k contiguous when B is transposed.
  const int vecA = aligned16(a.A, a.lda), vecB = aligned16(a.B, a.ldb);
  if (!a.transA && !a.transB)
    hipLaunchKernelGGL((gemm_f32_kernel<true, false>), grid, dim3(256), 0, s, a, tiles_n, vecA, vecB);
  else if (!a.transA && a.transB)
    hipLaunchKernelGGL((gemm_f32_kernel<true, true>), grid, dim3(256), 0, s, a, tiles_n, vecA, vecB);
  else if (a.transA && !a.transB)
    hipLaunchKernelGGL((gemm_f32_kernel<false, false>), grid, dim3(256), 0, s, a, tiles_n, vecA, vecB);
  else
    hipLaunchKernelGGL((gemm_f32_kernel<false, true>), grid, dim3(256), 0, s, a, tiles_n, vecA, vecB);
  return hipGetLastError();
}

}  // namespace gptq
