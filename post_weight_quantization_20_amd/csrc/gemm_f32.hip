// fp32 GEMM on CDNA4 matrix cores (v_mfma_f32_32x32x2_f32).
//
// Used for every dense fp32 product of the solver: the lazy-batch trailing update of the column
// loop (GPTQ tools page, "How it works", Step 7), the panel solves, symmetric rank-k updates and
// triangular-inverse products of the factor (Step 6), and the Hessian of fp32 activations (Step 3).
//
// A 256-thread workgroup (4 wave64s in a 2x2 grid) owns a T x T tile of C (T = 128: each wave holds
// 2x2 MFMA blocks of 32x32; T = 64: one block per wave). The reduction dimension is staged through LDS
// 32 at a time, double buffered, with the next stage's global loads in flight while the current
// stage feeds the MFMAs. An operand whose reduction index is contiguous in memory is kept
// row-major in LDS ([row][k]) and read with one 16-byte load per lane for four MFMAs, the lane's two
// k-halves taking k = 4h..4h+3 in turn; the other kind is kept k-major ([k][row]) and read 4 bytes
// per MFMA. Lower- or upper-triangle products launch only the tiles that touch the triangle.
#include "common.hpp"

#include <cmath>

namespace gptq {
namespace {

constexpr int GK = 32;   // k per LDS stage

template <int T, bool KC>
struct Stage {
  // LDS footprint of one operand stage, in floats
  static constexpr int ROWLEN = KC ? GK + 4 : T + 4;
  static constexpr int ROWS = KC ? T : GK;
  static constexpr int SIZE = ROWS * ROWLEN;
  static constexpr int NV = T * GK / 4 / 256;  // float4 per thread per stage
};

// Global -> registers -> LDS for one operand stage: logical element (k, r), k in [0, GK), r in [0, T).
// KC: stored matrix has k contiguous (P[r * ld + k]); otherwise r contiguous (P[k * ld + r]).
template <int T, bool KC>
struct Loader {
  using S = Stage<T, KC>;
  float4 v[S::NV];

  GPTQ_DEV static void coord(int idx, int& r, int& k) {
    if (KC) { r = idx / (GK / 4); k = (idx % (GK / 4)) * 4; }
    else    { k = idx / (T / 4);  r = (idx % (T / 4)) * 4; }
  }

  GPTQ_DEV void load(const float* __restrict__ P, int64_t ld, int64_t r0, int64_t R, int64_t k0, int64_t K,
                     bool vec, int tid) {
    if (vec && r0 + T <= R && k0 + GK <= K) {
#pragma unroll
      for (int i = 0; i < S::NV; ++i) {
        int r, k;
        coord(tid + i * 256, r, k);
        v[i] = KC ? *reinterpret_cast<const float4*>(P + (r0 + r) * ld + k0 + k)
                  : *reinterpret_cast<const float4*>(P + (k0 + k) * ld + r0 + r);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < S::NV; ++i) {
      int r, k;
      coord(tid + i * 256, r, k);
      float t[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t rr = r0 + r + (KC ? 0 : e), kk = k0 + k + (KC ? e : 0);
        t[e] = (rr < R && kk < K) ? (KC ? P[rr * ld + kk] : P[kk * ld + rr]) : 0.0f;
      }
      v[i] = make_float4(t[0], t[1], t[2], t[3]);
    }
  }

  GPTQ_DEV void store(float* Sm, int tid) const {
#pragma unroll
    for (int i = 0; i < S::NV; ++i) {
      int r, k;
      coord(tid + i * 256, r, k);
      if (KC) *reinterpret_cast<float4*>(Sm + r * S::ROWLEN + k) = v[i];
      else    *reinterpret_cast<float4*>(Sm + k * S::ROWLEN + r) = v[i];
    }
  }
};

// Operand values for four consecutive MFMAs (k = 4h + e of the current group of 8) of the block
// whose rows start at `row`.
template <int T, bool KC>
GPTQ_DEV float4 operand4(const float* Sm, int row, int kg, int lane) {
  using S = Stage<T, KC>;
  const int li = lane & 31, h = lane >> 5;
  if (KC) return *reinterpret_cast<const float4*>(Sm + (row + li) * S::ROWLEN + kg + 4 * h);
  return make_float4(Sm[(kg + 4 * h + 0) * S::ROWLEN + row + li], Sm[(kg + 4 * h + 1) * S::ROWLEN + row + li],
                     Sm[(kg + 4 * h + 2) * S::ROWLEN + row + li], Sm[(kg + 4 * h + 3) * S::ROWLEN + row + li]);
}

GPTQ_DEV float f4(const float4& v, int e) { return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w; }

// Tile t of a triangle of n x n tiles in row order: lower (tn <= tm) or upper (tn >= tm).
GPTQ_DEV void tri_tile(int64_t t, int64_t n, bool lower, int64_t& tm, int64_t& tn) {
  if (lower) {
    int64_t r = (int64_t)((sqrt(8.0 * (double)t + 1.0) - 1.0) * 0.5);
    while ((r + 1) * (r + 2) / 2 <= t) ++r;
    while (r * (r + 1) / 2 > t) --r;
    tm = r;
    tn = t - r * (r + 1) / 2;
  } else {
    // row r holds tiles (r, r..n-1): offset(r) = r n - r (r - 1) / 2
    int64_t r = 0, off = 0;
    // invert offset(r) <= t with a square root, then correct
    const double nn = (double)n + 0.5;
    r = (int64_t)(nn - sqrt(nn * nn - 2.0 * (double)t));
    if (r < 0) r = 0;
    while (r > 0 && r * n - r * (r - 1) / 2 > t) --r;
    while ((r + 1) * n - (r + 1) * r / 2 <= t) ++r;
    off = r * n - r * (r - 1) / 2;
    tm = r;
    tn = r + (t - off);
  }
}

template <int T, bool AK, bool BK>
__global__ __launch_bounds__(256, 2) void gemm_f32_kernel(GemmArgs a, int64_t tiles_n, int vecA, int vecB) {
  constexpr int WB = T / 64;  // 32x32 blocks per wave per dimension
  int64_t tm, tn;
  if (a.tri == 0) { tm = blockIdx.x / tiles_n; tn = blockIdx.x % tiles_n; }
  else tri_tile(blockIdx.x, tiles_n, a.tri == 1, tm, tn);
  const int64_t m0 = tm * T, n0 = tn * T;
  if (blockIdx.y > 0) {
    a.A += (int64_t)blockIdx.y * a.sA;
    a.B += (int64_t)blockIdx.y * a.sB;
    a.C += (int64_t)blockIdx.y * a.sC;
  }

  using SA = Stage<T, AK>;
  using SB = Stage<T, BK>;
  // the two operands' double-buffered stages, and after the loop the T x (T + 8) tile of results
  constexpr int TL = T + 8;
  constexpr int SMEM = std::max(2 * (SA::SIZE + SB::SIZE), T * TL);
  __shared__ __align__(16) float smem[SMEM];
  float (*As)[SA::SIZE] = reinterpret_cast<float (*)[SA::SIZE]>(smem);
  float (*Bs)[SB::SIZE] = reinterpret_cast<float (*)[SB::SIZE]>(smem + 2 * SA::SIZE);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int li = lane & 31, lk = lane >> 5;

  floatx16 acc[WB][WB];
#pragma unroll
  for (int i = 0; i < WB; ++i)
#pragma unroll
    for (int j = 0; j < WB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  Loader<T, AK> la;
  Loader<T, BK> lb;
  // a lower-triangular A is zero past the tile's last row (T is a multiple of GK)
  const int64_t kend = a.lowerA ? std::min<int64_t>(a.K, m0 + T) : a.K;
  const int64_t nk = (kend + GK - 1) / GK;
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
    // the operands of the next group of 8 k are read while the current group's MFMAs run
    float4 av[2][WB], bv[2][WB];
#pragma unroll
    for (int i = 0; i < WB; ++i) av[0][i] = operand4<T, AK>(As[cur], wm * (T / 2) + i * 32, 0, lane);
#pragma unroll
    for (int j = 0; j < WB; ++j) bv[0][j] = operand4<T, BK>(Bs[cur], wn * (T / 2) + j * 32, 0, lane);
#pragma unroll
    for (int g = 0; g < GK / 8; ++g) {
      const int c = g & 1;
      if (g + 1 < GK / 8) {
#pragma unroll
        for (int i = 0; i < WB; ++i) av[c ^ 1][i] = operand4<T, AK>(As[cur], wm * (T / 2) + i * 32, 8 * (g + 1), lane);
#pragma unroll
        for (int j = 0; j < WB; ++j) bv[c ^ 1][j] = operand4<T, BK>(Bs[cur], wn * (T / 2) + j * 32, 8 * (g + 1), lane);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int i = 0; i < WB; ++i)
#pragma unroll
          for (int j = 0; j < WB; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(f4(av[c][i], e), f4(bv[c][j], e), acc[i][j], 0, 0, 0);
    }
    // instruction order for the scheduler: the first two groups' LDS reads, then each group's MFMAs
    // followed by the reads of the group after next
    {
      constexpr int RA = AK ? WB : 4 * WB, RB = BK ? WB : 4 * WB;  // LDS reads per group, at most
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * (RA + RB), 0);
#pragma unroll
      for (int g = 0; g < GK / 8; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 4 * WB * WB, 0);
        if (g + 2 < GK / 8) __builtin_amdgcn_sched_group_barrier(0x100, RA + RB, 0);
      }
    }
    if (more) {
      la.store(As[cur ^ 1], tid);
      lb.store(Bs[cur ^ 1], tid);
    }
    __syncthreads();
  }

  // Epilogue through LDS (the stages are free after the loop's last barrier). Accumulator register
  // r of lane l holds row 8*(r/4) + 4*(l/32) + r%4, column l%32 of its 32x32 block; the rows of the
  // tile are padded to T + 8 floats so that the two half-waves' stores (4 rows apart) fall in
  // distinct banks. Then the workgroup reads C, adds and writes back along rows, each thread's loads
  // all in flight before its first store.
#pragma unroll
  for (int i = 0; i < WB; ++i)
#pragma unroll
    for (int j = 0; j < WB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        smem[(wm * (T / 2) + i * 32 + 8 * (r >> 2) + 4 * lk + (r & 3)) * TL + wn * (T / 2) + j * 32 + li] =
            a.alpha * acc[i][j][r];
  __syncthreads();
  const bool full = m0 + T <= a.M && n0 + T <= a.N && a.ldc % 4 == 0 && (uintptr_t)a.C % 16 == 0;
  if (full) {
    // 16-byte accesses; on a triangle's diagonal tile only the elements inside it are written
    constexpr int PT = T * T / 4 / 256;
    const bool whole = a.tri == 0 || (a.tri == 1 ? m0 >= n0 + T - 1 : m0 + T - 1 <= n0);
    float4 cv[PT];
    if (a.beta != 0.0f) {
#pragma unroll
      for (int q = 0; q < PT; ++q) {
        const int e = tid + q * 256, row = e / (T / 4), c4 = e % (T / 4) * 4;
        cv[q] = *reinterpret_cast<const float4*>(a.C + (m0 + row) * a.ldc + n0 + c4);
      }
    }
#pragma unroll
    for (int q = 0; q < PT; ++q) {
      const int e = tid + q * 256, row = e / (T / 4), c4 = e % (T / 4) * 4;
      float4 v = *reinterpret_cast<const float4*>(smem + row * TL + c4);
      if (a.beta != 0.0f) {
        v.x = __builtin_fmaf(a.beta, cv[q].x, v.x);
        v.y = __builtin_fmaf(a.beta, cv[q].y, v.y);
        v.z = __builtin_fmaf(a.beta, cv[q].z, v.z);
        v.w = __builtin_fmaf(a.beta, cv[q].w, v.w);
      }
      float* c = a.C + (m0 + row) * a.ldc + n0 + c4;
      if (whole) {
        *reinterpret_cast<float4*>(c) = v;
      } else {
        const int64_t m = m0 + row, n = n0 + c4;
        const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (a.tri == 1 ? m >= n + u : m <= n + u) c[u] = vv[u];
      }
    }
    return;
  }
  // a tile on the edge of C: element by element, 16 at a time, each group's loads first
  constexpr int PE = 16;
#pragma unroll 1
  for (int q0 = 0; q0 < T * T / 256; q0 += PE) {
    float cv[PE];
#pragma unroll
    for (int q = 0; q < PE; ++q) {
      const int e = tid + (q0 + q) * 256;
      const int64_t m = m0 + e / T, n = n0 + e % T;
      const bool in = m < a.M && n < a.N;
      cv[q] = (a.beta != 0.0f && in) ? a.C[m * a.ldc + n] : 0.0f;
    }
#pragma unroll
    for (int q = 0; q < PE; ++q) {
      const int e = tid + (q0 + q) * 256;
      const int64_t m = m0 + e / T, n = n0 + e % T;
      if (m >= a.M || n >= a.N) continue;
      if (a.tri == 1 && m < n) continue;
      if (a.tri == 2 && m > n) continue;
      const float v = smem[(e / T) * TL + e % T];
      a.C[m * a.ldc + n] = a.beta != 0.0f ? __builtin_fmaf(a.beta, cv[q], v) : v;
    }
  }
}

bool aligned16(const void* p, int64_t ld) { return ((uintptr_t)p % 16 == 0) && (ld % 4 == 0); }

template <int T>
hipError_t launch(const GemmArgs& a, hipStream_t s) {
  const int64_t tiles_m = (a.M + T - 1) / T, tiles_n = (a.N + T - 1) / T;
  int64_t tiles = tiles_m * tiles_n;
  int64_t tn_arg = tiles_n;
  if (a.tri != 0) {
    // square triangle of tiles (M == N for the symmetric products)
    tiles = tiles_n * (tiles_n + 1) / 2;
  }
  const unsigned nb = a.batch > 1 ? (unsigned)a.batch : 1u;
  const dim3 grid((unsigned)tiles, nb);
  // op(A) has k contiguous when A is not transposed; op(B) has k contiguous when B is transposed.
  const int vecA = aligned16(a.A, a.lda) && (nb == 1 || a.sA % 4 == 0);
  const int vecB = aligned16(a.B, a.ldb) && (nb == 1 || a.sB % 4 == 0);
  if (!a.transA && !a.transB)
    hipLaunchKernelGGL((gemm_f32_kernel<T, true, false>), grid, dim3(256), 0, s, a, tn_arg, vecA, vecB);
  else if (!a.transA && a.transB)
    hipLaunchKernelGGL((gemm_f32_kernel<T, true, true>), grid, dim3(256), 0, s, a, tn_arg, vecA, vecB);
  else if (a.transA && !a.transB)
    hipLaunchKernelGGL((gemm_f32_kernel<T, false, false>), grid, dim3(256), 0, s, a, tn_arg, vecA, vecB);
  else
    hipLaunchKernelGGL((gemm_f32_kernel<T, false, true>), grid, dim3(256), 0, s, a, tn_arg, vecA, vecB);
  return hipGetLastError();
}

}  // namespace

hipError_t gemm_f32(const GemmArgs& a, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (a.tri != 0 && a.M != a.N) return hipErrorInvalidValue;
  if (a.batch > 65535) return hipErrorInvalidValue;
  if (a.lowerA && a.transA) return hipErrorInvalidValue;
  // 128 x 128 tiles do more work per byte staged but run two to a CU (512 at a time on 256 CUs), so
  // they pay off when their count fills whole rounds of those slots, or when there are so many that
  // the last partial round hardly matters; otherwise 64 x 64 tiles (four times as many workgroups)
  // balance better. Measured on the solver's shapes (fp32, K = 128 and 512): with the q_proj lazy
  // product of N = 3072 (768 tiles, a round and a half) on 64 x 64 tiles, the layer's lazy products
  // took 0.651 instead of 0.682 ms (the two rules alternating in one process).
  const int64_t t128 = ((a.M + 127) / 128) * ((a.N + 127) / 128) / (a.tri ? 2 : 1) * std::max<int64_t>(a.batch, 1);
  if (t128 >= 4096 || (t128 >= 512 && t128 % 512 == 0)) return launch<128>(a, s);
  return launch<64>(a, s);
}

}  // namespace gptq
