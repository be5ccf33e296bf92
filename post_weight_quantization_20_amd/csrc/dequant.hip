// The stored layer at inference: y = x W^T for a few input rows, read straight from the packed codes.
//
// GPTQ tools page, "How it works", Step 8: after quantization a layer is kept as packed integer codes
// with a scale and zero point per group, and a fused kernel unpacks, scales and multiplies. What Is
// GPTQ ("How it works", Step 3) has each group expanded back to higher precision just in time for the
// matrix product; the pages' "Speed" note says small-batch inference is bound by reading the weights.
//
// W[r, k] = s[r, G(k)] * (q[r, k] - z[r, G(k)]), where q is nibble k % 8 of word k / 8 of row r and
// G(k) is g_idx[k], or k / g when no g_idx is given (groups of g consecutive columns).
//
// Two kernels:
//   dq_fast_kernel     fp16 x, groups of g consecutive columns with g % 32 == 0 (or one group per
//                      row), d % 32 == 0, 16-byte aligned rows of x. A lane takes 32 columns (one
//                      16-byte load per weight row) that share a group, so per lane and row
//                      sum_k x_k W[r,k] = s * (sum_k x_k q_k - z * sum_k x_k). The codes become
//                      exact fp16 integers with the 0x6400 exponent trick, and v_dot2_f32_f16 sums
//                      fp16 products (exact in fp32) into fp32. The sum of x over the 32 columns is
//                      shared by every weight row a wave holds.
//   dq_general_kernel  any x type, any g_idx: per column W[r, k] = s * (q - z) in fp32.
// Both are HBM-bound at small m: 0.5 byte of codes per weight against m FMAs.
#include <hip/hip_runtime.h>

#include "common.hpp"

namespace gptq {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

struct DqArgs {
  const void* x;
  int64_t ldx;
  int m;                      // rows of x in this pass (1..MT)
  const uint32_t* packed;     // rows x d/8 words
  int64_t rows, d;
  const float* scales;        // rows x ngroups
  const int32_t* zeros;       // rows x ngroups
  int64_t ngroups, g;
  uint32_t cpg;               // fast kernel: 32-column chunks per group (0: one group per row)
  const int32_t* gidx;        // null: G(k) = k / g
  float* y;                   // m x rows, row pitch ldy
  int64_t ldy;
};

// Sum over the 64 lanes of a wave, returned in every lane: DPP rotations inside each 16-lane row,
// then the four row sums read out with readlane.
GPTQ_DEV float wave_sum(float v) {
  v += row_ror<8>(v);
  v += row_ror<4>(v);
  v += row_ror<2>(v);
  v += row_ror<1>(v);
  const int b = __builtin_bit_cast(int, v);
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0)) +
         __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16)) +
         __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32)) +
         __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
}

GPTQ_DEV half2_t as_h2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }

// The eight codes of one word as four fp16 pairs (n_t, n_{t+4}), t = 0..3, exact small integers:
// OR-ing a nibble into the mantissa of 1024.0 (0x6400) gives 1024 + n; a nibble in bits 4..7 gives
// 1024 + 16 n, which times 1/16 minus 64 is n again. Both steps are exact in fp16.
GPTQ_DEV void decode_word(uint32_t w, half2_t (&q)[4]) {
  const half2_t m1024 = as_h2(0xE400E400u), r16 = as_h2(0x2C002C00u), m64 = as_h2(0xD400D400u);
  const uint32_t w8 = w >> 8;
  q[0] = as_h2((w & 0x000F000Fu) | 0x64006400u) + m1024;
  q[1] = as_h2((w & 0x00F000F0u) | 0x64006400u) * r16 + m64;
  q[2] = as_h2((w8 & 0x000F000Fu) | 0x64006400u) + m1024;
  q[3] = as_h2((w8 & 0x00F000F0u) | 0x64006400u) * r16 + m64;
}

// The matching fp16 pairs (x_t, x_{t+4}) of the eight inputs of one word's columns.
GPTQ_DEV void pair_inputs(u32x4 u, half2_t (&p)[4]) {
  p[0] = as_h2(__builtin_amdgcn_perm(u.z, u.x, 0x05040100u));
  p[1] = as_h2(__builtin_amdgcn_perm(u.z, u.x, 0x07060302u));
  p[2] = as_h2(__builtin_amdgcn_perm(u.w, u.y, 0x05040100u));
  p[3] = as_h2(__builtin_amdgcn_perm(u.w, u.y, 0x07060302u));
}

// Each wave holds R weight rows; four waves per workgroup. Lane l takes 32-column chunks l, l + 64, ...
template <int MT, int R>
__global__ __launch_bounds__(256) void dq_fast_kernel(DqArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t r0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * R;
  if (r0 >= a.rows) return;
  const int64_t nw = a.d >> 3, nv = nw >> 2;
  const u32x4* prow[R];
  const float* srow[R];
  const int32_t* zrow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t rr = min(r0 + r, a.rows - 1);
    prow[r] = reinterpret_cast<const u32x4*>(a.packed + rr * nw);
    srow[r] = a.scales + rr * a.ngroups;
    zrow[r] = a.zeros + rr * a.ngroups;
  }
  const u32x4* xrow[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
    xrow[i] = reinterpret_cast<const u32x4*>(static_cast<const _Float16*>(a.x) + (int64_t)min(i, a.m - 1) * a.ldx);
  const half2_t ones = as_h2(0x3C003C00u);

  float acc[MT][R];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[i][r] = 0.f;

  for (int64_t v = lane; v < nv; v += 64) {
    u32x4 w[R];
#pragma unroll
    for (int r = 0; r < R; ++r) w[r] = __builtin_nontemporal_load(prow[r] + v);
    const uint32_t grp = a.cpg ? (uint32_t)v / a.cpg : 0u;
    float s[R], z[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      s[r] = srow[r][grp];
      z[r] = (float)zrow[r][grp];
    }
    float inner[MT][R], sx[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      sx[i] = 0.f;
#pragma unroll
      for (int r = 0; r < R; ++r) inner[i][r] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      half2_t xp[MT][4];
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        pair_inputs(xrow[i][4 * v + j], xp[i]);
#pragma unroll
        for (int t = 0; t < 4; ++t) sx[i] = __builtin_amdgcn_fdot2(xp[i][t], ones, sx[i], false);
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const uint32_t word = w[r][j];
        half2_t q[4];
        decode_word(word, q);
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
          for (int t = 0; t < 4; ++t) inner[i][r] = __builtin_amdgcn_fdot2(xp[i][t], q[t], inner[i][r], false);
      }
    }
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int r = 0; r < R; ++r) acc[i][r] = __builtin_fmaf(s[r], __builtin_fmaf(-z[r], sx[i], inner[i][r]), acc[i][r]);
  }

#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float t = wave_sum(acc[i][r]);
      if (lane == 0 && i < a.m && r0 + r < a.rows) a.y[(int64_t)i * a.ldy + r0 + r] = t;
    }
}

template <int XT>
GPTQ_DEV float load_x(const void* x, int64_t idx) {
  if constexpr (XT == F32) return static_cast<const float*>(x)[idx];
  else if constexpr (XT == F16) return (float)static_cast<const _Float16*>(x)[idx];
  else return bf16_bits_to_f32(static_cast<const uint16_t*>(x)[idx]);
}

// Any input type and any column-to-group map. Lane l takes words l, l + 64, ... of R weight rows.
template <int XT, int MT, int R>
__global__ __launch_bounds__(256) void dq_general_kernel(DqArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t r0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * R;
  if (r0 >= a.rows) return;
  const int64_t nw = a.d >> 3;
  int64_t rr[R];
#pragma unroll
  for (int r = 0; r < R; ++r) rr[r] = min(r0 + r, a.rows - 1);
  float acc[MT][R];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[i][r] = 0.f;

  for (int64_t wv = lane; wv < nw; wv += 64) {
    uint32_t w[R];
#pragma unroll
    for (int r = 0; r < R; ++r) w[r] = a.packed[rr[r] * nw + wv];
    float xv[MT][8];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int t = 0; t < 8; ++t) xv[i][t] = load_x<XT>(a.x, (int64_t)min(i, a.m - 1) * a.ldx + 8 * wv + t);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int64_t k = 8 * wv + t;
      int64_t G = a.gidx ? (int64_t)a.gidx[k] : k / a.g;
      G = G < 0 ? 0 : G >= a.ngroups ? a.ngroups - 1 : G;   // out-of-range entries are clamped
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int32_t q = (int32_t)((w[r] >> (4 * t)) & 15u);
        const float wq = a.scales[rr[r] * a.ngroups + G] * (float)(q - a.zeros[rr[r] * a.ngroups + G]);
#pragma unroll
        for (int i = 0; i < MT; ++i) acc[i][r] = __builtin_fmaf(xv[i][t], wq, acc[i][r]);
      }
    }
  }

#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float t = wave_sum(acc[i][r]);
      if (lane == 0 && i < a.m && r0 + r < a.rows) a.y[(int64_t)i * a.ldy + r0 + r] = t;
    }
}

// Weight rows per wave: four when that still leaves at least 512 workgroups, else two, else one.
int rows_per_wave(int64_t rows) {
  if (rows >= 4 * 4 * 512) return 4;
  if (rows >= 2 * 4 * 512) return 2;
  return 1;
}

template <int MT, int R>
hipError_t launch_fast(const DqArgs& a, hipStream_t s) {
  const int64_t wgs = (a.rows + 4 * R - 1) / (4 * R);
  hipLaunchKernelGGL((dq_fast_kernel<MT, R>), dim3((unsigned)wgs), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int XT, int MT, int R>
hipError_t launch_general(const DqArgs& a, hipStream_t s) {
  const int64_t wgs = (a.rows + 4 * R - 1) / (4 * R);
  hipLaunchKernelGGL((dq_general_kernel<XT, MT, R>), dim3((unsigned)wgs), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int MT>
hipError_t dispatch_fast(const DqArgs& a, int R, hipStream_t s) {
  return R == 4 ? launch_fast<MT, 4>(a, s) : R == 2 ? launch_fast<MT, 2>(a, s) : launch_fast<MT, 1>(a, s);
}

template <int XT, int MT>
hipError_t dispatch_general(const DqArgs& a, int R, hipStream_t s) {
  return R == 4   ? launch_general<XT, MT, 4>(a, s)
         : R == 2 ? launch_general<XT, MT, 2>(a, s)
                  : launch_general<XT, MT, 1>(a, s);
}

template <int MT>
hipError_t dispatch(const DqArgs& a, int dtype, bool fast, int R, hipStream_t s) {
  if (fast) return dispatch_fast<MT>(a, R, s);
  if (dtype == F32) return dispatch_general<F32, MT>(a, R, s);
  if (dtype == F16) return dispatch_general<F16, MT>(a, R, s);
  return dispatch_general<BF16, MT>(a, R, s);
}

}  // namespace

bool dequant_fast_path(const void* x, int dtype, int64_t ldx, const int32_t* packed, const int32_t* gidx, int64_t d,
                       int64_t g) {
  return dtype == F16 && !gidx && d % 32 == 0 && (g >= d || g % 32 == 0) && ldx % 8 == 0 &&
         reinterpret_cast<uintptr_t>(x) % 16 == 0 && reinterpret_cast<uintptr_t>(packed) % 16 == 0;
}

hipError_t dequant_gemm(const void* x, int dtype, int64_t m, int64_t ldx, const int32_t* packed, const float* scales,
                        const int32_t* zeros, const int32_t* gidx, int64_t rows, int64_t d, int64_t g, float* y,
                        int64_t ldy, hipStream_t s) {
  const bool fast = dequant_fast_path(x, dtype, ldx, packed, gidx, d, g);
  const int R = rows_per_wave(rows);
  const int64_t esz = dtype == F32 ? 4 : 2;
  for (int64_t i0 = 0; i0 < m; i0 += 8) {
    DqArgs a{};
    a.x = static_cast<const char*>(x) + i0 * ldx * esz;
    a.ldx = ldx;
    a.m = (int)std::min<int64_t>(8, m - i0);
    a.packed = reinterpret_cast<const uint32_t*>(packed);
    a.rows = rows;
    a.d = d;
    a.scales = scales;
    a.zeros = zeros;
    a.g = g;
    a.ngroups = (d + g - 1) / g;
    a.cpg = g >= d ? 0u : (uint32_t)(g / 32);
    a.gidx = gidx;
    a.y = y + i0 * ldy;
    a.ldy = ldy;
    // weight rows per wave times input rows stays at most 8 (the accumulators' registers)
    hipError_t e = a.m == 1   ? dispatch<1>(a, dtype, fast, R, s)
                   : a.m == 2 ? dispatch<2>(a, dtype, fast, R, s)
                   : a.m <= 4 ? dispatch<4>(a, dtype, fast, std::min(R, 2), s)
                              : dispatch<8>(a, dtype, fast, 1, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace gptq
