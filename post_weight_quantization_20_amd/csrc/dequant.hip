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
// Three kernels, picked on the host:
//   dq_fast_kernel     one or two input rows (or more when the matrix-core kernel does not apply):
//                      fp16 x, groups of g consecutive columns with g % 32 == 0 (or one group per
//                      row), d % 32 == 0, 16-byte aligned rows of x and codes. A lane takes 32
//                      columns (one 16-byte load per weight row) that share a group, so per lane and
//                      row sum_k x_k W[r,k] = s * (sum_k x_k q_k - z * sum_k x_k). The codes become
//                      exact fp16 integers with the 0x6400 exponent trick, and v_dot2_f32_f16 sums
//                      fp16 products (exact in fp32) into fp32. The sum of x over the 32 columns is
//                      shared by every weight row a wave holds.
//   dq_mfma_kernel     3..16 input rows with the same layout conditions and g % 128 == 0: the same
//                      decoded codes feed v_mfma_f32_16x16x16f16, so the input rows cost no VALU.
//   dq_general_kernel  any x type, any g_idx (act-order), any g: per column W[r, k] = s * (q - z) in
//                      fp32, with the rows' (scale, zero) tables staged in LDS when they fit.
// At small m all three are bound by reading the codes: half a byte per weight against m FMAs.
#include <hip/hip_runtime.h>

#include "common.hpp"

namespace gptq {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct DqArgs {
  const void* x;
  int64_t ldx;
  int m;                      // rows of x in this pass (1..MT)
  const uint32_t* packed;     // rows x d/8 words
  int64_t rows, d;
  const float* scales;        // rows x ngroups
  const int32_t* zeros;       // rows x ngroups
  int64_t ngroups, g;
  uint32_t cpg;               // dot2 / matrix-core kernels: 32- or 128-column chunks per group (0: one group)
  const int32_t* gidx;        // null: G(k) = k / g
  int xvec;                   // general kernel: rows of x are 16-byte aligned (vector loads)
  int gvec;                   // general kernel: gidx is 16-byte aligned
  int bits;                   // code width
  int dense;                  // general kernel: 1 = dense bit stream, 0 = nibble / byte fields
  int64_t nwr;                // words per row of packed
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

// (w & mask) | magic in one v_and_or_b32. Written out because a VOP3 instruction takes no literal and
// one scalar operand here, so the compiler otherwise emits separate AND and OR instructions.
GPTQ_DEV uint32_t and_or(uint32_t w, uint32_t mask, uint32_t magic) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(w), "s"(mask), "v"(magic));
  return r;
}

// The eight codes of one word as four fp16 pairs (n_t, n_{t+4}), t = 0..3, exact small integers:
// OR-ing a nibble into the mantissa of 1024.0 (0x6400) gives 1024 + n; a nibble in bits 4..7 gives
// 1024 + 16 n, which times 1/16 minus 64 is n again. Both steps are exact in fp16.
GPTQ_DEV void decode_word(uint32_t w, half2_t (&q)[4]) {
  const half2_t m1024 = as_h2(0xE400E400u), r16 = as_h2(0x2C002C00u), m64 = as_h2(0xD400D400u);
  const uint32_t w8 = w >> 8;
  q[0] = as_h2(and_or(w, 0x000F000Fu, 0x64006400u)) + m1024;
  q[1] = as_h2(and_or(w, 0x00F000F0u, 0x64006400u)) * r16 + m64;
  q[2] = as_h2(and_or(w8, 0x000F000Fu, 0x64006400u)) + m1024;
  q[3] = as_h2(and_or(w8, 0x00F000F0u, 0x64006400u)) * r16 + m64;
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

  // the next chunk's codes, scales and zeros are loaded before the current chunk is computed
  // with one or two input rows, their 32 inputs are prefetched too
  constexpr bool kPreX = MT <= 2;
  // codes, scales and zeros of the next two chunks (and the next chunk's inputs) are in flight while
  // a chunk is computed
  u32x4 wn[R], wn2[R];
  float sn[R], sn2[R];
  int32_t zn[R], zn2[R];
  u32x4 xn[kPreX ? MT : 1][4];
  auto fetch_codes = [&](int64_t v, u32x4 (&w)[R], float (&sc)[R], int32_t (&zz)[R]) {
    const uint32_t grp = a.cpg ? (uint32_t)v / a.cpg : 0u;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      w[r] = __builtin_nontemporal_load(prow[r] + v);
      sc[r] = srow[r][grp];
      zz[r] = zrow[r][grp];
    }
  };
  auto fetch_inputs = [&](int64_t v) {
    if constexpr (kPreX) {
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) xn[i][j] = xrow[i][4 * v + j];
    }
  };
  if (lane < nv) {
    fetch_codes(lane, wn, sn, zn);
    fetch_inputs(lane);
  }
  if (lane + 64 < nv) fetch_codes(lane + 64, wn2, sn2, zn2);
  for (int64_t v = lane; v < nv; v += 64) {
    u32x4 w[R];
    float s[R], z[R];
    u32x4 xc[kPreX ? MT : 1][4];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      w[r] = wn[r];
      s[r] = sn[r];
      z[r] = (float)zn[r];
    }
    if constexpr (kPreX) {
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) xc[i][j] = xn[i][j];
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      wn[r] = wn2[r];
      sn[r] = sn2[r];
      zn[r] = zn2[r];
    }
    if (v + 128 < nv) fetch_codes(v + 128, wn2, sn2, zn2);
    if (v + 64 < nv) fetch_inputs(v + 64);
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
        if constexpr (kPreX) pair_inputs(xc[i][j], xp[i]);
        else pair_inputs(xrow[i][4 * v + j], xp[i]);
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

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));

// 3..16 input rows on the matrix cores. A workgroup owns 16 NT weight rows; its KS waves split the
// columns into 128-column units, four consecutive units (a quad) at a time (wave w takes quads
// w, w + KS, ...), each unit inside one group. A quad's codes are 256 contiguous bytes of each row:
// they are loaded four rows per instruction (16 bytes a lane along the run), which keeps the reads
// of HBM in long runs, and go through a padded, wave-private LDS area to the operand layout below
// (64-byte pieces of 16 rows per instruction streamed a third slower).
// v_mfma_f32_16x16x16f16 with A = x (16 input rows, rows >= m zero) and B = the codes as exact fp16
// integers accumulates T = sum x q over a unit; a second product with B = 1 gives sum x in the same
// lanes, and s (T - z sum x) is added per unit. Lane l holds B[k][j] and A[i][k] for j, i = l % 16 and
// k = 4 (l / 16) + 0..3; the k slots of lane group c = l / 16 map to the 32 columns c of the unit in
// the order (0,4,1,5), (2,6,3,7) of each word, which the decoded pairs and the permuted inputs share.
// The KS partial tiles are summed in LDS in wave order.
template <int KS, int NT>
__global__ __launch_bounds__(64 * KS) void dq_mfma_kernel(DqArgs a) {
  // a wave's staged quad: per tile 16 rows of 16 + 1 vectors of 16 bytes (the pad vector puts the
  // 16 rows' reads of one vector in distinct banks); after the loop the area holds the partial tiles
  constexpr int SROW = 17;
  constexpr int STAGE = 16 * SROW;
  __shared__ u32x4 stage[KS][NT][STAGE];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int jl = lane & 15, c = lane >> 4;
  // NT tiles of 16 weight rows share each unit's inputs (A operand) and its sum of x
  const int64_t j0 = (int64_t)blockIdx.x * 16 * NT;
  const float* srow[NT];
  const int32_t* zrow[NT];
  const int64_t nw = a.d >> 3;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int64_t row = min(j0 + 16 * t + jl, a.rows - 1);
    srow[t] = a.scales + row * a.ngroups;
    zrow[t] = a.zeros + row * a.ngroups;
  }
  const bool xval = jl < a.m;
  const u32x4* xr = reinterpret_cast<const u32x4*>(static_cast<const _Float16*>(a.x) + (int64_t)min(jl, a.m - 1) * a.ldx);
  const uint32_t units = (uint32_t)(a.d >> 7);
  const half4_t ones = {(_Float16)1, (_Float16)1, (_Float16)1, (_Float16)1};
  const half2_t m1024 = as_h2(0xE400E400u), r16 = as_h2(0x2C002C00u), m64 = as_h2(0xD400D400u);

  floatx4 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = floatx4{0.f, 0.f, 0.f, 0.f};
  // A 128-column unit u: this lane's codes are words 16u + 4c .. +3 of its rows and its inputs
  // columns 128u + 32c .. +31 of input row l % 16; one scale and zero per unit and row.
  struct Codes {
    u32x4 w[NT];
    float sc[NT];
    int32_t z[NT];
  };
  struct Inputs {
    u32x4 x[4];
  };
  auto load_inputs = [&](uint32_t u, Inputs& in) {
#pragma unroll
    for (int q = 0; q < 4; ++q) in.x[q] = xval ? xr[16 * (int64_t)u + 4 * c + q] : u32x4{0u, 0u, 0u, 0u};
  };
  auto unit = [&](const Codes& cd, const Inputs& in) {
    floatx4 T[NT], S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < NT; ++t) T[t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      half2_t p[4];
      pair_inputs(in.x[q], p);
      const half4_t a0 = __builtin_shufflevector(p[0], p[1], 0, 1, 2, 3);
      const half4_t a1 = __builtin_shufflevector(p[2], p[3], 0, 1, 2, 3);
      S = __builtin_amdgcn_mfma_f32_16x16x16f16(a0, ones, S, 0, 0, 0);
      S = __builtin_amdgcn_mfma_f32_16x16x16f16(a1, ones, S, 0, 0, 0);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const uint32_t wd = cd.w[t][q], w8 = wd >> 8;
        const half2_t q0 = as_h2(and_or(wd, 0x000F000Fu, 0x64006400u)) + m1024;
        const half2_t q1 = as_h2(and_or(wd, 0x00F000F0u, 0x64006400u)) * r16 + m64;
        const half2_t q2 = as_h2(and_or(w8, 0x000F000Fu, 0x64006400u)) + m1024;
        const half2_t q3 = as_h2(and_or(w8, 0x00F000F0u, 0x64006400u)) * r16 + m64;
        T[t] = __builtin_amdgcn_mfma_f32_16x16x16f16(a0, __builtin_shufflevector(q0, q1, 0, 1, 2, 3), T[t], 0, 0, 0);
        T[t] = __builtin_amdgcn_mfma_f32_16x16x16f16(a1, __builtin_shufflevector(q2, q3, 0, 1, 2, 3), T[t], 0, 0, 0);
      }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float z = (float)cd.z[t];
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[t][r] = __builtin_fmaf(cd.sc[t], __builtin_fmaf(-z, S[r], T[t][r]), acc[t][r]);
    }
  };

  // The wave's units in order: the four of quad w, then those of quad w + KS, and so on. When a quad
  // starts, its codes (loaded one quad earlier) go to LDS and the wave's next quad is loaded; the
  // metadata and inputs of each unit are loaded two units ahead.
  const uint32_t quads = (units + 3) / 4;
  const uint32_t nvec = 4 * units;   // 16-byte vectors of codes in a row
  u32x4 raw[NT][4];
  auto load_quad = [&](uint32_t q) {
    const uint32_t v = 16 * q + (uint32_t)(lane & 15);
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t row = min(j0 + 16 * t + 4 * i + (lane >> 4), a.rows - 1);
        raw[t][i] = v < nvec ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.packed + row * nw) + v)
                             : u32x4{0u, 0u, 0u, 0u};
      }
  };
  auto store_quad = [&]() {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) stage[wave][t][(4 * i + (lane >> 4)) * SROW + (lane & 15)] = raw[t][i];
  };
  auto load_meta = [&](uint32_t u, Codes& cd) {
    const uint32_t grp = a.cpg ? u / a.cpg : 0u;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      cd.sc[t] = srow[t][grp];
      cd.z[t] = zrow[t][grp];
    }
  };
  auto next_unit = [&](uint32_t u) { return (u & 3u) != 3u && u + 1 < units ? u + 1 : (u & ~3u) + 4 * KS; };
  uint32_t u = 4 * (uint32_t)wave;
  uint32_t u1 = next_unit(u);
  Codes cn, cn2;
  Inputs xn, xn2;
  if (u < units) {
    load_quad((uint32_t)wave);
    load_meta(u, cn);
    load_inputs(u, xn);
  }
  if (u1 < units) {
    load_meta(u1, cn2);
    load_inputs(u1, xn2);
  }
  while (u < units) {
    if ((u & 3u) == 0) {
      store_quad();
      const uint32_t qn = u / 4 + KS;
      if (qn < quads) load_quad(qn);
    }
    Codes cd = cn;
    const Inputs xi = xn;
#pragma unroll
    for (int t = 0; t < NT; ++t) cd.w[t] = stage[wave][t][jl * SROW + 4 * (int)(u & 3u) + c];
    cn = cn2;
    xn = xn2;
    const uint32_t u2 = u1 < units ? next_unit(u1) : u1;
    if (u2 < units) {
      load_meta(u2, cn2);
      load_inputs(u2, xn2);
    }
    unit(cd, xi);
    u = u1;
    u1 = u2;
  }
  __syncthreads();   // every wave is done with its stage area, which now takes the partial tiles
  floatx4 (*part)[NT][64] = reinterpret_cast<floatx4 (*)[NT][64]>(&stage[0][0][0]);
#pragma unroll
  for (int t = 0; t < NT; ++t) part[wave][t][lane] = acc[t];
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      floatx4 sum = part[0][t][lane];
#pragma unroll
      for (int w = 1; w < KS; ++w) {
        const floatx4 o = part[w][t][lane];
#pragma unroll
        for (int r = 0; r < 4; ++r) sum[r] += o[r];
      }
      const int64_t j = j0 + 16 * t + jl;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * c + r;
        if (i < a.m && j < a.rows) a.y[(int64_t)i * a.ldy + j] = sum[r];
      }
    }
  }
}

template <int XT>
GPTQ_DEV float load_x(const void* x, int64_t idx) {
  if constexpr (XT == F32) return static_cast<const float*>(x)[idx];
  else if constexpr (XT == F16) return (float)static_cast<const _Float16*>(x)[idx];
  else return bf16_bits_to_f32(static_cast<const uint16_t*>(x)[idx]);
}

// The codes of columns 8 wv .. 8 wv + 7 of one row. Fields: one word of nibbles (bits <= 4) or two
// words of bytes. Dense stream: the 8 bits-wide codes start at stream bit 8 wv bits and span at most
// three words (8 bits <= 64 bits from an offset below 32).
template <bool NIB>
GPTQ_DEV void codes8(const uint32_t* __restrict__ row, int64_t nwr, int64_t wv, int bits, int dense,
                     uint32_t (&q)[8]) {
  if (NIB) {
    const uint32_t w = row[wv];
#pragma unroll
    for (int t = 0; t < 8; ++t) q[t] = (w >> (4 * t)) & 15u;
    return;
  }
  if (!dense) {
    if (bits <= 4) {
      const uint32_t w = row[wv];
#pragma unroll
      for (int t = 0; t < 8; ++t) q[t] = (w >> (4 * t)) & 15u;
    } else {
      const uint32_t w0 = row[2 * wv], w1 = row[2 * wv + 1];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        q[t] = (w0 >> (8 * t)) & 255u;
        q[4 + t] = (w1 >> (8 * t)) & 255u;
      }
    }
    return;
  }
  const int64_t b0 = 8 * wv * bits;
  const int64_t w0 = b0 >> 5;
  const int off = (int)(b0 & 31);
  const uint32_t a0 = row[w0];
  const uint32_t a1 = w0 + 1 < nwr ? row[w0 + 1] : 0u;
  const uint32_t a2 = w0 + 2 < nwr ? row[w0 + 2] : 0u;
  // the 96-bit window a2:a1:a0 shifted right by off, as two 64-bit halves
  const uint64_t lo = ((uint64_t)a1 << 32) | a0, hi = a2;
  const uint64_t win = off ? (lo >> off) | (hi << (64 - off)) : lo;   // bits off .. off + 63
  const uint32_t mask = (1u << bits) - 1u;
#pragma unroll
  for (int t = 0; t < 8; ++t) q[t] = (uint32_t)(win >> (t * bits)) & mask;
}

// x[row][8 wv .. 8 wv + 7] as floats: one or two 16-byte loads when the rows are 16-byte aligned.
template <int XT>
GPTQ_DEV void load_x8(const void* x, int64_t base, bool vec, float (&v)[8]) {
  if (vec) {
    if constexpr (XT == F32) {
      const floatx4 a = *reinterpret_cast<const floatx4*>(static_cast<const float*>(x) + base);
      const floatx4 b = *reinterpret_cast<const floatx4*>(static_cast<const float*>(x) + base + 4);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        v[t] = a[t];
        v[4 + t] = b[t];
      }
    } else {
      const u32x4 u = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) + base);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t lo = u[t] & 0xFFFFu, hi = u[t] >> 16;
        if constexpr (XT == F16) {
          v[2 * t] = (float)__builtin_bit_cast(_Float16, (uint16_t)lo);
          v[2 * t + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)hi);
        } else {
          v[2 * t] = __builtin_bit_cast(float, lo << 16);
          v[2 * t + 1] = __builtin_bit_cast(float, hi << 16);
        }
      }
    }
  } else {
#pragma unroll
    for (int t = 0; t < 8; ++t) v[t] = load_x<XT>(x, base + t);
  }
}

// Any input type and any column-to-group map. Lane l takes words l, l + 64, ... of R weight rows.
// With TAB the workgroup's rows' (scale, zero) tables are first copied to LDS, so that each weight
// reads its group's pair with one LDS load instead of two global gathers. NIB: nibble fields (the
// common layout, decoded without the layout tests).
template <int XT, int MT, int R, bool TAB, bool NIB>
__global__ __launch_bounds__(256) void dq_general_kernel(DqArgs a) {
  extern __shared__ u32x2 tab[];   // [4 R][ngroups]: scale bits, zero
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t rb = (int64_t)blockIdx.x * 4 * R;
  if constexpr (TAB) {
    const int64_t n = 4 * R * a.ngroups;
    for (int64_t i = threadIdx.x; i < n; i += 256) {
      const int64_t wr = i / a.ngroups, G = i - wr * a.ngroups;
      const int64_t row = min(rb + wr, a.rows - 1);
      u32x2 e;
      e.x = __builtin_bit_cast(uint32_t, a.scales[row * a.ngroups + G]);
      e.y = (uint32_t)a.zeros[row * a.ngroups + G];
      tab[i] = e;
    }
    __syncthreads();
  }
  const int64_t r0 = rb + (int64_t)wave * R;
  if (r0 >= a.rows) return;
  const int64_t nw = a.d >> 3;
  int64_t rr[R];
#pragma unroll
  for (int r = 0; r < R; ++r) rr[r] = min(r0 + r, a.rows - 1);
  const bool xvec = a.xvec != 0;
  float acc[MT][R];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[i][r] = 0.f;

  for (int64_t wv = lane; wv < nw; wv += 64) {
    uint32_t qc[R][8];
#pragma unroll
    for (int r = 0; r < R; ++r) codes8<NIB>(a.packed + rr[r] * a.nwr, a.nwr, wv, a.bits, a.dense, qc[r]);
    int32_t gk[8];
    if (a.gidx && a.gvec) {
      const u32x4 g0 = *reinterpret_cast<const u32x4*>(a.gidx + 8 * wv);
      const u32x4 g1 = *reinterpret_cast<const u32x4*>(a.gidx + 8 * wv + 4);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        gk[t] = (int32_t)g0[t];
        gk[4 + t] = (int32_t)g1[t];
      }
    } else if (a.gidx) {
#pragma unroll
      for (int t = 0; t < 8; ++t) gk[t] = a.gidx[8 * wv + t];
    } else {
#pragma unroll
      for (int t = 0; t < 8; ++t) gk[t] = (int32_t)((8 * wv + t) / a.g);
    }
    float xv[MT][8];
#pragma unroll
    for (int i = 0; i < MT; ++i) load_x8<XT>(a.x, (int64_t)min(i, a.m - 1) * a.ldx + 8 * wv, xvec, xv[i]);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int64_t G = gk[t] < 0 ? 0 : gk[t] >= a.ngroups ? a.ngroups - 1 : gk[t];   // clamped
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int32_t q = (int32_t)qc[r][t];
        float sc;
        int32_t z;
        if constexpr (TAB) {
          const u32x2 e = tab[(wave * R + r) * a.ngroups + G];
          sc = __builtin_bit_cast(float, e.x);
          z = (int32_t)e.y;
        } else {
          sc = a.scales[rr[r] * a.ngroups + G];
          z = a.zeros[rr[r] * a.ngroups + G];
        }
        const float wq = sc * (float)(q - z);
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
  const int64_t tab_bytes = 4 * R * a.ngroups * (int64_t)sizeof(u32x2);
  const bool nib = !a.dense && a.bits <= 4;
  if (tab_bytes <= 65536) {
    if (nib)
      hipLaunchKernelGGL((dq_general_kernel<XT, MT, R, true, true>), dim3((unsigned)wgs), dim3(256), (size_t)tab_bytes,
                         s, a);
    else
      hipLaunchKernelGGL((dq_general_kernel<XT, MT, R, true, false>), dim3((unsigned)wgs), dim3(256),
                         (size_t)tab_bytes, s, a);
  } else {
    if (nib)
      hipLaunchKernelGGL((dq_general_kernel<XT, MT, R, false, true>), dim3((unsigned)wgs), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((dq_general_kernel<XT, MT, R, false, false>), dim3((unsigned)wgs), dim3(256), 0, s, a);
  }
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

// The matrix-core kernel: fp16 inputs, groups of whole 128-column units, aligned rows.
bool dequant_mfma_path(const void* x, int dtype, int64_t ldx, const int32_t* packed, const int32_t* gidx, int64_t d,
                       int64_t g) {
  return dtype == F16 && !gidx && d % 128 == 0 && (g >= d || g % 128 == 0) && ldx % 8 == 0 &&
         reinterpret_cast<uintptr_t>(x) % 16 == 0 && reinterpret_cast<uintptr_t>(packed) % 16 == 0;
}

bool dequant_fast_path(const void* x, int dtype, int64_t ldx, const int32_t* packed, const int32_t* gidx, int64_t d,
                       int64_t g) {
  return dtype == F16 && !gidx && d % 32 == 0 && (g >= d || g % 32 == 0) && ldx % 8 == 0 &&
         reinterpret_cast<uintptr_t>(x) % 16 == 0 && reinterpret_cast<uintptr_t>(packed) % 16 == 0;
}

}  // namespace

hipError_t dequant_gemm(const void* x, int dtype, int64_t m, int64_t ldx, const int32_t* packed, int bits, int dense,
                        const float* scales, const int32_t* zeros, const int32_t* gidx, int64_t rows, int64_t d,
                        int64_t g, float* y, int64_t ldy, hipStream_t s) {
  // the dot2 and matrix-core kernels decode nibble fields; other layouts take the general kernel
  const bool nibbles = !dense && bits <= 4;
  const bool fast = nibbles && dequant_fast_path(x, dtype, ldx, packed, gidx, d, g);
  // two input rows still run faster on the dot2 kernel (fc2: 90 against 108 us); three or more do not
  const bool mfma = nibbles && m >= 3 && dequant_mfma_path(x, dtype, ldx, packed, gidx, d, g);
  const int R = rows_per_wave(rows);
  const int64_t esz = dtype == F32 ? 4 : 2;
  const int64_t step = mfma ? 16 : 8;
  for (int64_t i0 = 0; i0 < m; i0 += step) {
    DqArgs a{};
    a.x = static_cast<const char*>(x) + i0 * ldx * esz;
    a.ldx = ldx;
    a.m = (int)std::min<int64_t>(step, m - i0);
    a.packed = reinterpret_cast<const uint32_t*>(packed);
    a.rows = rows;
    a.d = d;
    a.scales = scales;
    a.zeros = zeros;
    a.g = g;
    a.ngroups = (d + g - 1) / g;
    a.gidx = gidx;
    a.y = y + i0 * ldy;
    a.ldy = ldy;
    a.bits = bits;
    a.dense = dense;
    a.nwr = dense ? d * bits / 32 : bits <= 4 ? d / 8 : d / 4;
    hipError_t e;
    if (mfma && a.m >= 3) {
      // units per group; waves per workgroup so that about 12 waves per CU are in flight
      a.cpg = g >= d ? 0u : (uint32_t)(g / 128);
      const int64_t tiles = (rows + 15) / 16;
      if (tiles >= 768 && a.m > 4) {
        // two 16-row tiles per wave share the inputs; 8 waves split the columns (with four inputs
        // or fewer, one tile a wave and two workgroups a CU run faster: fc2 117 against 122 us)
        hipLaunchKernelGGL((dq_mfma_kernel<8, 2>), dim3((unsigned)((tiles + 1) / 2)), dim3(512), 0, s, a);
      } else {
        hipLaunchKernelGGL((dq_mfma_kernel<8, 1>), dim3((unsigned)tiles), dim3(512), 0, s, a);
      }
      e = hipGetLastError();
    } else {
      a.cpg = fast && g < d ? (uint32_t)(g / 32) : 0u;
      a.xvec = ldx % (dtype == F32 ? 4 : 8) == 0 && reinterpret_cast<uintptr_t>(a.x) % 16 == 0;
      a.gvec = gidx && reinterpret_cast<uintptr_t>(gidx) % 16 == 0;
      // weight rows per wave times input rows stays at most 8 (the accumulators' registers)
      e = a.m == 1   ? dispatch<1>(a, dtype, fast, R, s)
          : a.m == 2 ? dispatch<2>(a, dtype, fast, R, s)
          : a.m <= 4 ? dispatch<4>(a, dtype, fast, std::min(R, 2), s)
                     : dispatch<8>(a, dtype, fast, 1, s);
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace gptq
