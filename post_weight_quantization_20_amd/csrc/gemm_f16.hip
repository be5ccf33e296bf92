// fp16 GEMM C = alpha A B^T + beta C on CDNA4 matrix cores (v_mfma_f32_32x32x16_f16), and the
// two-term fp16 split that lets it stand in for an fp32 product.
//
// A [M x K] and B [N x K] are fp16, row-major with k contiguous; products are exact in fp32 and sums
// are fp32. A 1024-thread workgroup (16 wave64s in a 4x4 grid) owns a 256 x 256 tile of C, each wave
// 2x2 blocks of 32x32 (the kernel takes the wave grid, the blocks per wave and the stage depth as
// parameters). K is staged through LDS 64 at a time, double buffered: lane l reads 8
// consecutive k of row l % 32 (k = 8 (l / 32) .. +7 of each 16-wide step) with one 16-byte LDS read
// per operand block. Tiles run in groups of 16 row tiles by every column tile, row tile fastest, so
// the workgroups in flight share a few A strips and every B strip through L2 and the Infinity Cache.
//
// The split: x = hi + lo with hi = fp16(x) and lo = fp16(x - hi), exact to within 2^-22 |x| (2^-25
// absolute where lo is subnormal). An fp32 product x . w is then hi_x hi_w + hi_x lo_w + lo_x hi_w up
// to the dropped lo_x lo_w (below 2^-22 |x w|): the rows of A become [hi | hi | lo] and those of B
// [hi | lo | hi], each padded with zeros to a multiple of 64, and one fp16 GEMM over 3d forms the sum.
// Weights are scaled by a power of two before the split, so that their lo parts stay normal fp16;
// alpha undoes it exactly.
#include "common.hpp"

namespace gptq {
namespace {

constexpr int HK = 64;         // K granularity of the operands (the deepest LDS stage)
constexpr int HGROUP = 16;     // row tiles per group

// A wave owns BM x BN blocks of 32x32; WGM x WGN waves (tile 32 BM WGM x 32 BN WGN); K is staged KS at
// a time.
template <int WGM, int WGN, int BM, int BN, int KS>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_f16nt_kernel(GemmF16 a, int64_t tiles_m, int64_t tiles_n) {
  constexpr int NTH = 64 * WGM * WGN;
  constexpr int TM = 32 * BM * WGM, TN = 32 * BN * WGN, ROW = KS + 8, PQ = KS / 8;
  constexpr int PA = TM * KS / 8 / NTH, PB = TN * KS / 8 / NTH;   // 16-byte pieces per thread
  // grouped order: group g covers row tiles [16 g, 16 g + 16) and every column tile
  const int64_t per_group = (int64_t)HGROUP * tiles_n;
  const int64_t g = blockIdx.x / per_group, in = blockIdx.x % per_group;
  const int64_t first = g * HGROUP;
  const int64_t gm = min((int64_t)HGROUP, tiles_m - first);
  const int64_t tm = first + in % gm, tn = in / gm;
  const int64_t m0 = tm * TM, n0 = tn * TN;
  if (a.lower && n0 > m0 + TM - 1) return;   // the whole workgroup leaves together
  if (blockIdx.y > 0) {
    a.A += (int64_t)blockIdx.y * a.sA;
    a.B += (int64_t)blockIdx.y * a.sB;
    a.C += (int64_t)blockIdx.y * a.sC;
  }

  __shared__ __align__(16) _Float16 As[2][TM * ROW];
  __shared__ __align__(16) _Float16 Bs[2][TN * ROW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int li = lane & 31, lh = lane >> 5;

  floatx16 acc[BM][BN];
#pragma unroll
  for (int i = 0; i < BM; ++i)
#pragma unroll
    for (int j = 0; j < BN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // global -> registers: piece p of an operand stage is row p / PQ, halves 8 (p % PQ) .. +7. Rows
  // past M or N read as zeros.
  u32x4 ra[PA], rb[PB];
  auto gload = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < PA; ++i) {
      const int p = tid + NTH * i, r = p / PQ, kq = p % PQ;
      const int64_t mr = m0 + r;
      ra[i] = mr < a.M ? *reinterpret_cast<const u32x4*>(a.A + mr * a.lda + k0 + 8 * kq) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < PB; ++i) {
      const int p = tid + NTH * i, r = p / PQ, kq = p % PQ;
      const int64_t nr = n0 + r;
      rb[i] = nr < a.N ? *reinterpret_cast<const u32x4*>(a.B + nr * a.ldb + k0 + 8 * kq) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PA; ++i) {
      const int p = tid + NTH * i, r = p / PQ, kq = p % PQ;
      *reinterpret_cast<u32x4*>(&As[buf][r * ROW + 8 * kq]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < PB; ++i) {
      const int p = tid + NTH * i, r = p / PQ, kq = p % PQ;
      *reinterpret_cast<u32x4*>(&Bs[buf][r * ROW + 8 * kq]) = rb[i];
    }
  };

  const int64_t nk = a.K / KS;
  if (nk > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int cur = (int)(kt & 1);
    const bool more = kt + 1 < nk;
    if (more) gload((kt + 1) * KS);
#pragma unroll
    for (int ks = 0; ks < KS; ks += 16) {
      half8 av[BM], bv[BN];
#pragma unroll
      for (int i = 0; i < BM; ++i)
        av[i] = *reinterpret_cast<const half8*>(&As[cur][(wm * 32 * BM + i * 32 + li) * ROW + ks + 8 * lh]);
#pragma unroll
      for (int j = 0; j < BN; ++j)
        bv[j] = *reinterpret_cast<const half8*>(&Bs[cur][(wn * 32 * BN + j * 32 + li) * ROW + ks + 8 * lh]);
#pragma unroll
      for (int i = 0; i < BM; ++i)
#pragma unroll
        for (int j = 0; j < BN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j], acc[i][j], 0, 0, 0);
    }
    if (more) lstore(cur ^ 1);
    __syncthreads();
  }

  // accumulator register r of lane l: row 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32 of its block
#pragma unroll
  for (int i = 0; i < BM; ++i)
#pragma unroll
    for (int j = 0; j < BN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * 32 * BM + i * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
        const int64_t n = n0 + wn * 32 * BN + j * 32 + li;
        if (m < a.M && n < a.N) {
          float* c = a.C + m * a.ldc + n;
          float v = a.alpha * acc[i][j][r];
          if (a.beta != 0.0f) v = __builtin_fmaf(a.beta, *c, v);
          *c = v;
        }
      }
}

template <int WGM, int WGN, int BM, int BN, int KS>
hipError_t launch_f16nt(const GemmF16& a, hipStream_t s) {
  constexpr int TM = 32 * BM * WGM, TN = 32 * BN * WGN;
  const int64_t tiles_m = (a.M + TM - 1) / TM, tiles_n = (a.N + TN - 1) / TN;
  if (tiles_m * tiles_n > 0x7fffffff) return hipErrorInvalidValue;
  const unsigned nb = a.batch > 1 ? (unsigned)a.batch : 1u;
  hipLaunchKernelGGL((gemm_f16nt_kernel<WGM, WGN, BM, BN, KS>), dim3((unsigned)(tiles_m * tiles_n), nb),
                     dim3(64 * WGM * WGN), 0, s, a, tiles_m, tiles_n);
  return hipGetLastError();
}

// Row t of X [n x d] (pitch ldx) -> row t of S [n x kp] (pitch kp): [hi | hi | lo | 0] (act) or
// [hi | lo | hi | 0] (!act) of scale * x. Thread k of a row reads x[k] once and writes its three
// copies; the kp - 3d padding columns are zeroed by the first threads. Rows stride by gridDim.y.
__global__ __launch_bounds__(256) void split3_kernel(const float* __restrict__ X, int64_t n, int64_t d, int64_t ldx,
                                                     float scale, int act, int64_t kp, _Float16* __restrict__ S) {
  const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t pad = kp - 3 * d;
  for (int64_t t = blockIdx.y; t < n; t += gridDim.y) {
    _Float16* row = S + t * kp;
    if (k < d) {
      const float x = scale * X[t * ldx + k];
      const _Float16 hi = (_Float16)x, lo = (_Float16)(x - (float)hi);
      row[k] = hi;
      row[d + k] = act ? hi : lo;
      row[2 * d + k] = act ? lo : hi;
    }
    if (k < pad) row[3 * d + k] = (_Float16)0.0f;
  }
}

// Per-workgroup maxima of |x| over n floats (grid-stride), then one workgroup folds them.
__global__ __launch_bounds__(256) void absmax_partial_kernel(const float* __restrict__ x, int64_t n,
                                                             float* __restrict__ part) {
  __shared__ float red[4];
  float m = 0.0f;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256)
    m = fmaxf(m, fabsf(x[e]));
#pragma unroll
  for (int s = 32; s > 0; s >>= 1) m = fmaxf(m, __shfl_xor(m, s, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) part[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__global__ __launch_bounds__(256) void absmax_final_kernel(const float* __restrict__ part, int np,
                                                           float* __restrict__ out) {
  __shared__ float red[4];
  float m = 0.0f;
  for (int i = threadIdx.x; i < np; i += 256) m = fmaxf(m, part[i]);
#pragma unroll
  for (int s = 32; s > 0; s >>= 1) m = fmaxf(m, __shfl_xor(m, s, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) out[0] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

}  // namespace

hipError_t gemm_f16nt(const GemmF16& a, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (a.K % HK != 0 || a.lda % 8 != 0 || a.ldb % 8 != 0 || (uintptr_t)a.A % 16 != 0 || (uintptr_t)a.B % 16 != 0)
    return hipErrorInvalidValue;
  if (a.batch > 65535 || (a.batch > 1 && (a.sA % 8 != 0 || a.sB % 8 != 0))) return hipErrorInvalidValue;
  // 16 waves in a 4x4 grid, 2x2 blocks each: a 256 x 256 tile with a 64-deep stage (147 KB of LDS),
  // one workgroup (four waves per SIMD) per CU. Measured on the Llama-7B block's products: 6% faster
  // than a 32-deep stage, which was about 5% faster than 4-wave 128 x 128 tiles (and 1-3% faster
  // than 8-wave 256 x 128 or 128 x 256 tiles); 4-wave tiles with 4x2 or 2x4 blocks per wave (one wave
  // per SIMD) were 12-25% slower than the 128 x 128 ones.
  return launch_f16nt<4, 4, 2, 2, 64>(a, s);
}

int64_t split3_pitch(int64_t d) { return (3 * d + HK - 1) / HK * HK; }

hipError_t split3(const float* X, int64_t n, int64_t d, int64_t ldx, float scale, int act, _Float16* S,
                  hipStream_t s) {
  const int64_t kp = split3_pitch(d);
  if (n <= 0 || d <= 0) return hipSuccess;
  const int64_t cols = std::max(d, kp - 3 * d);
  hipLaunchKernelGGL(split3_kernel, dim3((unsigned)((cols + 255) / 256), (unsigned)std::min<int64_t>(n, 65535)),
                     dim3(256), 0, s, X, n, d, ldx, scale, act, kp, S);
  return hipGetLastError();
}

hipError_t absmax(const float* x, int64_t n, float* part, float* out, hipStream_t s) {
  const int np = (int)std::min<int64_t>(std::max<int64_t>((n + 255) / 256, 1), kAbsmaxParts);
  hipLaunchKernelGGL(absmax_partial_kernel, dim3((unsigned)np), dim3(256), 0, s, x, n, part);
  hipLaunchKernelGGL(absmax_final_kernel, dim3(1), dim3(256), 0, s, part, np, out);
  return hipGetLastError();
}

}  // namespace gptq
