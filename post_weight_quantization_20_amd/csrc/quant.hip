// The GPTQ column loop with lazy block updates, and the nibble packer.
//
// GPTQ tools page, "How it works":
//   Step 5 - columns are quantized one at a time in a fixed order; each column's rounding error,
//            divided by the matching diagonal entry of the factor, is subtracted from the columns
//            not yet quantized through the matching row of the factor;
//   Step 7 - columns are processed in blocks; inside a block updates are applied at once, updates to
//            later columns are collected and applied once when the block ends (lazy batch);
//   Step 8 - one scale and zero point per group of weights; codes packed eight 4-bit values per word.
// "What Is GPTQ?" (ai-tldr.dev), "How it works", Step 3: groups are runs of consecutive weights of a
// row, each with its own scale and zero point.
//
// Rows of W are independent once U is known, so the block kernel gives each row 16 lanes of a
// wave64 (4 rows per wave, 16 rows per 256-thread workgroup). A lane holds B/16 consecutive columns
// of its row in registers; the block's part of U sits in LDS, and the row of U for column k is read
// by all rows of the workgroup at once. Column k's weight is broadcast from its owning lane to the
// 16 lanes of its row with a DPP row broadcast, every lane then runs the rounding chain, and each lane
// applies the update to its own columns. Group minima and maxima are butterfly reductions across the
// 16 lanes. The block's scaled errors go to a rows x B buffer that the trailing update (an fp32 MFMA
// GEMM) multiplies into the columns after the block.
#include "common.hpp"

namespace gptq {
namespace {

struct QArgs {
  float* Wp;             // working weights, processing order, [rows x ldw]
  int64_t ldw;
  int64_t rows, d;
  int64_t b;             // first column of the block
  int ncols;             // columns in this block (<= 16 * CPL)
  const float* U;        // [d x d], processing order
  int64_t g;             // group size (columns)
  int grid_in_block;     // groups start inside blocks (g <= B); else the grid was computed for the block
  float maxq;
  uint8_t* codes_p;      // [rows x d], processing order
  float* scales;         // [rows x ngroups]
  int32_t* zeros;        // [rows x ngroups]
  int64_t ngroups;
  int sym;               // symmetric grids (in-block grids only)
  int compact;           // 16-bit scales, zeros clamped to the code width (in-block grids only)
  const int32_t* colgrp; // static groups: group of each processing column (its grid is in scales/zeros)
  float* err;            // this block's errors: [rows x 16 * CPL] at leading dimension err_ld
  int64_t err_ld;
  double* row_loss;      // [rows]
};

// Loads N consecutive floats from LDS (16-byte aligned when N >= 4) into registers.
template <int N>
GPTQ_DEV void lds_load(const float* p, float (&v)[N]) {
  if constexpr (N >= 4) {
#pragma unroll
    for (int i = 0; i < N; i += 4) {
      const float4 q = *reinterpret_cast<const float4*>(p + i);
      v[i] = q.x; v[i + 1] = q.y; v[i + 2] = q.z; v[i + 3] = q.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = p[i];
  }
}

// STATIC: every column takes the grid of its static group, colgrp[b + k] (loaded one chunk ahead with
// U's rows); no grid is computed here.
template <int CPL, bool STATIC>
__global__ __launch_bounds__(256) void quant_block_kernel(QArgs a) {
  constexpr int BP = 16 * CPL;
  extern __shared__ float sm[];
  float* Us = sm;                  // [BP][BP]: strict upper part of U's block, zeros elsewhere
  float* invd = Us + BP * BP;      // [BP]: 1 / U[k][k]
  float* Es = invd + BP;           // [16 rows][BP]: scaled errors of the block
  uint8_t* Qs = reinterpret_cast<uint8_t*>(Es + 16 * BP);  // [16 rows][BP]: codes of the block

  const int tid = threadIdx.x;
  const int nc = a.ncols;
  const int lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15;
  const int rloc = wave * 4 + (lane >> 4);
  const int64_t row = (int64_t)blockIdx.x * 16 + rloc;
  const bool row_ok = row < a.rows;

  // lane lr starts with block columns lr*CPL .. lr*CPL+CPL-1 in w[0..CPL-1] (read first, so that
  // these loads overlap the staging of U's block)
  float w[CPL];
  const float* wrow = a.Wp + row * a.ldw + a.b;
#pragma unroll
  for (int c = 0; c < CPL; ++c) w[c] = (row_ok && lr * CPL + c < nc) ? wrow[lr * CPL + c] : 0.0f;

  bool filled = false;
  if constexpr (CPL >= 4) {
   if (nc == BP && a.d % 4 == 0 && a.b % 4 == 0) {
    // full block: unconditional 16-byte loads, all in flight together
    filled = true;
    constexpr int Q = BP / 4;  // float4 per row
    float4 v[BP * Q / 256];
#pragma unroll
    for (int i = 0; i < BP * Q / 256; ++i) {
      const int e = tid + i * 256, k = e / Q, j = (e % Q) * 4;
      v[i] = *reinterpret_cast<const float4*>(a.U + (a.b + k) * a.d + a.b + j);
    }
#pragma unroll
    for (int i = 0; i < BP * Q / 256; ++i) {
      const int e = tid + i * 256, k = e / Q, j = (e % Q) * 4;
      float4 u = v[i];
      u.x = (j + 0 > k) ? u.x : 0.0f;
      u.y = (j + 1 > k) ? u.y : 0.0f;
      u.z = (j + 2 > k) ? u.z : 0.0f;
      u.w = (j + 3 > k) ? u.w : 0.0f;
      *reinterpret_cast<float4*>(Us + k * BP + j) = u;
    }
   }
  }
  if (!filled) {
    for (int e = tid; e < BP * BP; e += 256) {
      const int k = e / BP, j = e % BP;
      Us[e] = (j > k && j < nc) ? a.U[(a.b + k) * a.d + a.b + j] : 0.0f;
    }
  }
  for (int k = tid; k < BP; k += 256) invd[k] = (k < nc) ? 1.0f / a.U[(a.b + k) * a.d + a.b + k] : 0.0f;
  __syncthreads();

  float s = 1.0f, z = 0.0f, rs = 1.0f;
  if (!STATIC && !a.grid_in_block) {
    const int64_t gi = a.b / a.g;
    if (row_ok) {
      s = a.scales[row * a.ngroups + gi];
      z = (float)a.zeros[row * a.ngroups + gi];
    }
    rs = 1.0f / s;
  }
  float loss = 0.0f;
  // groups nest inside blocks when g <= B, so they start at block columns 0, g, 2g, ...
  int next_group = (!STATIC && a.grid_in_block) ? 0 : (1 << 30);
  const int gsz = (int)min<int64_t>(a.g, (int64_t)BP);

  // Chunk o quantizes block columns o*CPL .. o*CPL+CPL-1. Before it, the lanes of each row have
  // been rotated o times by one lane, so lane 0 holds those columns and lane l holds the columns
  // of original lane (l + o) mod 16 (already quantized ones meet zeros in U and stay unchanged).
  // What a chunk reads from LDS (U's rows for its columns, their reciprocal diagonal) is read one
  // chunk ahead, into the other of two register sets; U and the diagonal are not written after the
  // barrier above, and the chunk's own stores go to the codes and errors.
  const int nchunks = (nc + CPL - 1) / CPL;
  // static groups: the scale and zero of each of a chunk's columns (one chunk ahead, like U's rows)
  float sA[STATIC ? CPL : 1], zA[STATIC ? CPL : 1], sB[STATIC ? CPL : 1], zB[STATIC ? CPL : 1];
  auto fetch_grid = [&](int o, float (&sv)[STATIC ? CPL : 1], float (&zv)[STATIC ? CPL : 1]) {
    if constexpr (STATIC) {
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const int k = min(o * CPL + c, nc - 1);
        const int64_t G = a.colgrp[a.b + k];
        sv[c] = row_ok ? a.scales[row * a.ngroups + G] : 1.0f;
        zv[c] = row_ok ? (float)a.zeros[row * a.ngroups + G] : 0.0f;
      }
    }
  };
  auto fetch = [&](int o, float (&iv)[CPL], float (&ur)[CPL][CPL]) {
    const int cbase = ((lr + o) & 15) * CPL;
    lds_load<CPL>(invd + o * CPL, iv);
#pragma unroll
    for (int c = 0; c < CPL; ++c) lds_load<CPL>(Us + (o * CPL + c) * BP + cbase, ur[c]);
  };
  // CHECKS: the chunk may start a group or run past the block's last column (a plain chunk, full
  // and without a group start, runs the column chain with no branch or select)
  auto chunk = [&](int o, const float (&iv)[CPL], const float (&ur)[CPL][CPL], const float (&sv)[STATIC ? CPL : 1],
                   const float (&zv)[STATIC ? CPL : 1], auto checks) {
    constexpr bool CHECKS = decltype(checks)::value;
    const int cbase = ((lr + o) & 15) * CPL;  // block column of w[0] in this lane
    float qv[CPL], ev[CPL];
    float rsv[STATIC ? CPL : 1];
    if constexpr (STATIC) {
#pragma unroll
      for (int c = 0; c < CPL; ++c) rsv[c] = 1.0f / sv[c];
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int k = o * CPL + c;
      if constexpr (STATIC) {
        s = sv[c];
        z = zv[c];
        rs = rsv[c];
      }
      if (CHECKS && k == next_group) {
        next_group += gsz;
        // group grid from the current weights of block columns [k, k + g); min and max over the
        // row's 16 lanes by DPP rotations
        const int kend = min(k + gsz, nc);
        float mn = INFINITY, mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < CPL; ++t) {
          const int col = cbase + t;
          if (col >= k && col < kend) { mn = fminf(mn, w[t]); mx = fmaxf(mx, w[t]); }
        }
        mn = fminf(mn, row_ror<8>(mn)); mx = fmaxf(mx, row_ror<8>(mx));
        mn = fminf(mn, row_ror<4>(mn)); mx = fmaxf(mx, row_ror<4>(mx));
        mn = fminf(mn, row_ror<2>(mn)); mx = fmaxf(mx, row_ror<2>(mx));
        mn = fminf(mn, row_ror<1>(mn)); mx = fmaxf(mx, row_ror<1>(mx));
        make_grid(mn, mx, a.maxq, a.sym != 0, a.compact != 0, s, z, rs);
        if (lr == 0 && row_ok && k < nc) {
          // column and group indices stay below 2^31
          const int64_t gi = (uint32_t)(a.b + k) / (uint32_t)a.g;
          a.scales[row * a.ngroups + gi] = s;
          a.zeros[row * a.ngroups + gi] = (int32_t)z;
        }
      }
      // q = clamp(rint(w / s) + z, 0, maxq) and the value s (q - z). On the chain: q - z is
      // rint(w / s) clamped to [-z, maxq - z] (exact in fp32: small integers), and w - s (q - z) is
      // one fused multiply-add.
      const float wk = row_bcast<0>(w[c]);
      const float x = div_rn(wk, s, rs);
      const float qd = __builtin_amdgcn_fmed3f(rintf(x), -z, a.maxq - z);
      const float q = qd + z;
      float e = __builtin_fmaf(-s, qd, wk) * iv[c];
      if (CHECKS) e = (k < nc) ? e : 0.0f;
      loss = __builtin_fmaf(e, e, loss);
#pragma unroll
      for (int t = 0; t < CPL; ++t) w[t] = __builtin_fmaf(-e, ur[c][t], w[t]);
      qv[c] = q;
      ev[c] = e;
    }
    if (lr == 0) {
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        Qs[rloc * BP + o * CPL + c] = (uint8_t)qv[c];
        Es[rloc * BP + o * CPL + c] = ev[c];
      }
    }
#pragma unroll
    for (int t = 0; t < CPL; ++t) w[t] = row_ror15(w[t]);
  };
  auto run = [&](int o, const float (&iv)[CPL], const float (&ur)[CPL][CPL], const float (&sv)[STATIC ? CPL : 1],
                 const float (&zv)[STATIC ? CPL : 1]) {
    if (o * CPL + CPL <= nc && next_group >= o * CPL + CPL) chunk(o, iv, ur, sv, zv, std::false_type{});
    else chunk(o, iv, ur, sv, zv, std::true_type{});
  };
  float ivA[CPL], urA[CPL][CPL], ivB[CPL], urB[CPL][CPL];
  if (nchunks > 0) {
    fetch(0, ivA, urA);
    fetch_grid(0, sA, zA);
  }
  for (int o = 0; o < nchunks; o += 2) {
    if (o + 1 < nchunks) {
      fetch(o + 1, ivB, urB);
      fetch_grid(o + 1, sB, zB);
    }
    run(o, ivA, urA, sA, zA);
    if (o + 1 < nchunks) {
      if (o + 2 < nchunks) {
        fetch(o + 2, ivA, urA);
        fetch_grid(o + 2, sA, zA);
      }
      run(o + 1, ivB, urB, sB, zB);
    }
  }
  __syncthreads();

  if (row_ok) {
    uint8_t* crow = a.codes_p + row * a.d + a.b;
    float* erow = a.err + row * a.err_ld;
    const int j0 = lr * CPL;
    const bool vec = CPL == 8 && nc == BP && a.d % 8 == 0 && a.b % 8 == 0 && a.err_ld % 4 == 0 &&
                     (uintptr_t)a.codes_p % 8 == 0 && (uintptr_t)a.err % 16 == 0;
    if constexpr (CPL == 8) {
      if (vec) {
        *reinterpret_cast<uint2*>(crow + j0) = *reinterpret_cast<const uint2*>(Qs + rloc * BP + j0);
        *reinterpret_cast<float4*>(erow + j0) = *reinterpret_cast<const float4*>(Es + rloc * BP + j0);
        *reinterpret_cast<float4*>(erow + j0 + 4) = *reinterpret_cast<const float4*>(Es + rloc * BP + j0 + 4);
      }
    }
    if (!(CPL == 8 && vec)) {
#pragma unroll
      for (int t = 0; t < CPL; ++t) {
        const int j = j0 + t;
        if (j < nc) crow[j] = Qs[rloc * BP + j];
        erow[j] = (j < nc) ? Es[rloc * BP + j] : 0.0f;
      }
    }
    if (lr == 0) a.row_loss[row] += (double)loss;
  }
}

// Group grid for groups longer than a block: min/max of the current weights of columns
// [b, b + len) of each row, one wave per row.
__global__ __launch_bounds__(256) void group_grid_kernel(const float* __restrict__ Wp, int64_t ldw, int64_t rows,
                                                         int64_t b, int64_t len, float maxq, int sym, int compact,
                                                         int64_t gi,
                                                         float* __restrict__ scales, int32_t* __restrict__ zeros,
                                                         int64_t ngroups) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const float* p = Wp + row * ldw + b;
  float mn = INFINITY, mx = -INFINITY;
  for (int64_t j = lane; j < len; j += 64) {
    const float v = p[j];
    mn = fminf(mn, v);
    mx = fmaxf(mx, v);
  }
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) {
    mn = fminf(mn, __shfl_xor(mn, m, 64));
    mx = fmaxf(mx, __shfl_xor(mx, m, 64));
  }
  if (lane == 0) {
    float s, z, rs;
    make_grid(mn, mx, maxq, sym != 0, compact != 0, s, z, rs);
    scales[row * ngroups + gi] = s;
    zeros[row * ngroups + gi] = (int32_t)z;
  }
}

// Static groups: the grid of group G of every row from the original weights W[row][G g .. G g + g),
// one wave per (row, group); before any column is quantized.
__global__ __launch_bounds__(256) void static_grid_kernel(const void* __restrict__ W, int dtype, int64_t ld_w,
                                                          int64_t rows, int64_t d, int64_t g, int64_t ngroups,
                                                          float maxq, int sym, int compact,
                                                          float* __restrict__ scales, int32_t* __restrict__ zeros) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= rows * ngroups) return;
  const int64_t row = item / ngroups, G = item - row * ngroups;
  const int64_t c0 = G * g, c1 = min(c0 + g, d);
  float mn = INFINITY, mx = -INFINITY;
  for (int64_t j = c0 + lane; j < c1; j += 64) {
    const float v = load_as_f32(W, dtype, row * ld_w + j);
    mn = fminf(mn, v);
    mx = fmaxf(mx, v);
  }
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) {
    mn = fminf(mn, __shfl_xor(mn, m, 64));
    mx = fmaxf(mx, __shfl_xor(mx, m, 64));
  }
  if (lane == 0) {
    float s, z, rs;
    make_grid(mn, mx, maxq, sym != 0, compact != 0, s, z, rs);
    scales[item] = s;
    zeros[item] = (int32_t)z;
  }
}

// Working copy in processing order: Wp[r][j] = W[r][perm[j]] as fp32; zero padding to ldw (a
// multiple of 4). A thread writes four consecutive columns, as one 16-byte store when Wp allows.
__global__ __launch_bounds__(256) void gather_w_kernel(const void* __restrict__ W, int dtype, int64_t ldw_in,
                                                       int64_t rows, int64_t d, const int32_t* __restrict__ perm,
                                                       float* __restrict__ Wp, int64_t ldw, int vec) {
  for (int64_t r = blockIdx.y; r < rows; r += gridDim.y)
    for (int64_t j = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4; j < ldw; j += (int64_t)gridDim.x * 1024) {
      float v[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) v[t] = (j + t < d) ? load_as_f32(W, dtype, r * ldw_in + perm[j + t]) : 0.0f;
      float* o = Wp + r * ldw + j;
      if (vec) {
        *reinterpret_cast<float4*>(o) = make_float4(v[0], v[1], v[2], v[3]);
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) o[t] = v[t];
      }
    }
}

// iperm[perm[j]] = j, and g_idx[perm[j]] = j / g; with static groups g_idx[j] = j / g and
// colgrp[j] = perm[j] / g, the group whose grid processing column j takes.
__global__ void index_kernel(const int32_t* __restrict__ perm, int64_t d, int64_t g, int32_t* __restrict__ iperm,
                             int32_t* __restrict__ g_idx, int32_t* __restrict__ colgrp) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j < d) {
    const int32_t c = perm[j];
    iperm[c] = (int32_t)j;
    if (colgrp) {
      g_idx[j] = (int32_t)(j / g);
      colgrp[j] = (int32_t)(c / g);
    } else {
      g_idx[c] = (int32_t)(j / g);
    }
  }
}

// codes[r][c] = codes_p[r][iperm[c]] (back to the original column order). A thread writes four
// consecutive codes, as one 4-byte store when the row allows.
__global__ __launch_bounds__(256) void unpermute_kernel(const uint8_t* __restrict__ codes_p, int64_t rows, int64_t d,
                                                        const int32_t* __restrict__ iperm, uint8_t* __restrict__ codes,
                                                        int vec) {
  for (int64_t r = blockIdx.y; r < rows; r += gridDim.y)
    for (int64_t c = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4; c < d; c += (int64_t)gridDim.x * 1024) {
      const uint8_t* src = codes_p + r * d;
      uint8_t* dst = codes + r * d + c;
      if (vec && c + 4 <= d) {
        const uint32_t w = src[iperm[c]] | (src[iperm[c + 1]] << 8) | (src[iperm[c + 2]] << 16) |
                           ((uint32_t)src[iperm[c + 3]] << 24);
        *reinterpret_cast<uint32_t*>(dst) = w;
      } else {
        for (int64_t t = 0; t < 4 && c + t < d; ++t) dst[t] = src[iperm[c + t]];
      }
    }
}

__global__ void zero_f64(double* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.0;
}

// loss = sum of the row losses in a fixed order.
__global__ __launch_bounds__(1024) void loss_kernel(const double* __restrict__ row_loss, int64_t rows,
                                                    double* __restrict__ loss) {
  __shared__ double part[1024];
  double acc = 0.0;
  for (int64_t i = threadIdx.x; i < rows; i += 1024) acc += row_loss[i];
  part[threadIdx.x] = acc;
  __syncthreads();
  for (int s = 512; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) part[threadIdx.x] += part[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) *loss = part[0];
}

// Byte fields (codes of 5 to 8 bits): word k of a row holds columns 4k .. 4k + 3 in bytes 0..3,
// which is the code array's own byte order, so the words are a copy of the codes.
__global__ __launch_bounds__(256) void pack_bytes_kernel(const uint8_t* __restrict__ codes, int64_t n,
                                                         uint8_t* __restrict__ packed, int vec) {
  const int64_t n16 = vec ? n / 16 : 0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256)
    reinterpret_cast<uint4*>(packed)[i] = reinterpret_cast<const uint4*>(codes)[i];
  for (int64_t i = n16 * 16 + (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    packed[i] = codes[i];
}

// Dense bit stream: code k of a row takes stream bits bits k .. bits k + bits - 1 and stream bit t is
// bit t % 32 of word t / 32. One thread per output word ORs in every code that overlaps it.
__global__ __launch_bounds__(256) void pack_dense_kernel(const uint8_t* __restrict__ codes, int64_t rows, int64_t d,
                                                         int bits, int32_t* __restrict__ packed) {
  const int64_t words = d * bits / 32;
  const int64_t total = rows * words;
  const uint32_t mask = (1u << bits) - 1u;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / words, w = i % words;
    const int64_t b0 = 32 * w;
    const int64_t k0 = b0 / bits, k1 = min((b0 + 31) / bits, d - 1);
    const uint8_t* p = codes + r * d;
    uint32_t out = 0;
    for (int64_t k = k0; k <= k1; ++k) {
      const int64_t pos = k * bits - b0;   // in (-bits, 32)
      const uint32_t v = p[k] & mask;
      out |= pos >= 0 ? (v << pos) : (v >> -pos);
    }
    packed[i] = (int32_t)out;
  }
}

// Codes in processing order: column j of the output is column order[j] of the codes, packed in the
// field layout (nibbles up to 4 bits, bytes above). One thread per output word.
__global__ __launch_bounds__(256) void pack_ordered_kernel(const uint8_t* __restrict__ codes, int64_t rows, int64_t d,
                                                           const int32_t* __restrict__ order, int bits,
                                                           int32_t* __restrict__ packed) {
  const int f = bits <= 4 ? 4 : 8, per = 32 / f;
  const uint32_t mask = (1u << f) - 1u;
  const int64_t words = d / per;
  const int64_t total = rows * words;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / words, k = i % words;
    const uint8_t* p = codes + r * d;
    uint32_t out = 0;
    for (int t = 0; t < per; ++t) {
      const int64_t c = min(max((int64_t)order[per * k + t], (int64_t)0), d - 1);   // clamped into the row
      out |= ((uint32_t)p[c] & mask) << (f * t);
    }
    packed[i] = (int32_t)out;
  }
}

// Columns of a row-major matrix gathered by an order: out[i][j] = in[i][order[j]], elements of esz
// bytes (2 or 4).
__global__ __launch_bounds__(256) void permute_columns_kernel(const void* __restrict__ in, int64_t m, int64_t d,
                                                              int64_t ld_in, const int32_t* __restrict__ order,
                                                              int esz, void* __restrict__ out, int64_t ld_out) {
  const int64_t total = m * d;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int64_t i = e / d, j = e % d;
    const int64_t c = min(max((int64_t)order[j], (int64_t)0), d - 1);   // clamped into the row
    const int64_t src = i * ld_in + c, dst = i * ld_out + j;
    if (esz == 2) static_cast<uint16_t*>(out)[dst] = static_cast<const uint16_t*>(in)[src];
    else static_cast<uint32_t*>(out)[dst] = static_cast<const uint32_t*>(in)[src];
  }
}

// packed[r][k] = sum_t (codes[r][8k + t] & 15) << 4t.
__global__ __launch_bounds__(256) void pack_kernel(const uint8_t* __restrict__ codes, int64_t rows, int64_t d,
                                                   int32_t* __restrict__ packed, int vec) {
  const int64_t words = d / 8;
  const int64_t total = rows * words;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / words, k = i % words;
    const uint8_t* p = codes + r * d + 8 * k;
    uint32_t lo, hi;
    if (vec) {
      const uint2 v = *reinterpret_cast<const uint2*>(p);
      lo = v.x; hi = v.y;
    } else {
      lo = p[0] | (p[1] << 8) | (p[2] << 16) | ((uint32_t)p[3] << 24);
      hi = p[4] | (p[5] << 8) | (p[6] << 16) | ((uint32_t)p[7] << 24);
    }
    // byte t of lo/hi -> nibble t / t + 4
    uint32_t out = 0;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      out |= ((lo >> (8 * t)) & 15u) << (4 * t);
      out |= ((hi >> (8 * t)) & 15u) << (4 * (t + 4));
    }
    packed[i] = (int32_t)out;
  }
}

template <int CPL>
size_t qsmem() {
  constexpr size_t BP = 16 * CPL;
  return (BP * BP + BP + 16 * BP) * sizeof(float) + 16 * BP;
}

template <int CPL, bool STATIC>
void launch_block(const QArgs& a, hipStream_t s) {
  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute((const void*)quant_block_kernel<CPL, STATIC>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)qsmem<CPL>());
    attr = true;
  }
  hipLaunchKernelGGL((quant_block_kernel<CPL, STATIC>), dim3((unsigned)((a.rows + 15) / 16)), dim3(256), qsmem<CPL>(),
                     s, a);
}

template <int CPL>
void launch_block(const QArgs& a, bool is_static, hipStream_t s) {
  if (is_static) launch_block<CPL, true>(a, s);
  else launch_block<CPL, false>(a, s);
}

int cpl_for(int B) { return B <= 16 ? 1 : B <= 32 ? 2 : B <= 64 ? 4 : 8; }
int64_t super_width_max(int B) { return std::max<int64_t>(1, 512 / B) * B; }

}  // namespace

// Width of a super-block: the lazy updates of a block reach only the rest of its super-block, and
// the columns beyond are updated once per super-block (a product over the super-block's width
// instead of one per block). A group wider than a block reads columns that still lack the
// super-block's deferred updates unless groups and super-blocks nest, so the width is chosen to
// nest with such groups (a single group per row starts before any update and needs nothing).
int64_t super_width(int B, int64_t g, int64_t d) {
  for (int64_t m = std::max<int64_t>(1, 512 / B); m >= 1; --m) {
    const int64_t sw = m * B;
    if (g <= B || g >= d || sw % g == 0 || g % sw == 0) return sw;
  }
  return B;
}

QuantLayout quant_layout(int64_t rows, int64_t d, int block) {
  QuantLayout L;
  L.ldw = (d + 3) / 4 * 4;
  L.bp = 16 * cpl_for(block);
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  size_t o = 0;
  L.off_wp = o; o = up(o + (size_t)rows * L.ldw * sizeof(float));
  L.off_codes = o; o = up(o + (size_t)rows * d);
  // errors of one super-block (the last block writes up to bp columns past its start)
  L.ld_err = (super_width_max(block) + L.bp + 3) / 4 * 4;
  L.off_err = o; o = up(o + (size_t)rows * L.ld_err * sizeof(float));
  L.off_loss = o; o = up(o + (size_t)rows * sizeof(double));
  L.off_iperm = o; o = up(o + (size_t)d * sizeof(int32_t));
  L.off_colgrp = o; o = up(o + (size_t)d * sizeof(int32_t));
  L.total = o;
  return L;
}

hipError_t quantize(const void* W, int w_dtype, int64_t rows, int64_t d, int64_t ld_w, const float* U,
                    const int32_t* perm, int bits, int64_t g, int B, int sym, int static_groups, int compact,
                    uint8_t* codes, float* scales, int32_t* zeros, int32_t* g_idx, double* loss, void* work,
                    hipStream_t s) {
  const QuantLayout L = quant_layout(rows, d, B);
  char* wb = static_cast<char*>(work);
  float* Wp = reinterpret_cast<float*>(wb + L.off_wp);
  uint8_t* codes_p = reinterpret_cast<uint8_t*>(wb + L.off_codes);
  float* err = reinterpret_cast<float*>(wb + L.off_err);
  double* row_loss = reinterpret_cast<double*>(wb + L.off_loss);
  int32_t* iperm = reinterpret_cast<int32_t*>(wb + L.off_iperm);
  int32_t* colgrp = static_groups ? reinterpret_cast<int32_t*>(wb + L.off_colgrp) : nullptr;
  const int64_t ngroups = (d + g - 1) / g;
  const float maxq = (float)((1 << bits) - 1);

  hipLaunchKernelGGL(index_kernel, dim3((unsigned)((d + 255) / 256)), dim3(256), 0, s, perm, d, g, iperm, g_idx,
                     colgrp);
  if (static_groups && rows > 0) {
    const int64_t items = rows * ngroups;
    hipLaunchKernelGGL(static_grid_kernel, dim3((unsigned)((items + 3) / 4)), dim3(256), 0, s, W, w_dtype, ld_w, rows,
                       d, g, ngroups, maxq, sym, compact, scales, zeros);
  }
  if (rows > 0) {
    const unsigned gx = (unsigned)std::min<int64_t>((L.ldw + 1023) / 1024, 64);
    const int vec = (uintptr_t)Wp % 16 == 0;
    hipLaunchKernelGGL(gather_w_kernel, dim3(gx, (unsigned)std::min<int64_t>(rows, 65535)), dim3(256), 0, s, W, w_dtype,
                       ld_w, rows, d, perm, Wp, L.ldw, vec);
    hipLaunchKernelGGL(zero_f64, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s, row_loss, rows);
  }
  hipError_t e;
  const int cpl = cpl_for(B);
  const int64_t sw = super_width(B, g, d);
  GemmArgs t{};  // W[:, c0:c1] -= Err U[rows of the errors, c0:c1]
  t.M = rows; t.transA = 0; t.ldb = d; t.transB = 0; t.ldc = L.ldw;
  t.alpha = -1.0f; t.beta = 1.0f; t.tri = 0; t.lda = L.ld_err;
  for (int64_t s0 = 0; s0 < d && rows > 0; s0 += sw) {
    const int64_t s1 = std::min(d, s0 + sw);
    for (int64_t b = s0; b < s1; b += B) {
      const int nc = (int)std::min<int64_t>(B, d - b);
      const bool in_block = g <= B;
      if (!static_groups && !in_block && b % g == 0) {
        hipLaunchKernelGGL(group_grid_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, Wp, L.ldw, rows, b,
                           std::min<int64_t>(g, d - b), maxq, sym, compact, b / g, scales, zeros, ngroups);
      }
      QArgs a;
      a.Wp = Wp; a.ldw = L.ldw; a.rows = rows; a.d = d; a.b = b; a.ncols = nc; a.U = U; a.g = g;
      a.grid_in_block = in_block; a.maxq = maxq; a.codes_p = codes_p; a.scales = scales; a.zeros = zeros;
      a.ngroups = ngroups; a.err = err + (b - s0); a.err_ld = L.ld_err; a.row_loss = row_loss;
      a.sym = sym; a.compact = compact; a.colgrp = colgrp;
      const bool st = static_groups != 0;
      switch (cpl) {
        case 1: launch_block<1>(a, st, s); break;
        case 2: launch_block<2>(a, st, s); break;
        case 4: launch_block<4>(a, st, s); break;
        default: launch_block<8>(a, st, s); break;
      }
      if (b + nc < s1) {  // lazy batch inside the super-block
        t.N = s1 - b - nc; t.K = nc;
        t.A = err + (b - s0); t.B = U + b * d + b + nc; t.C = Wp + b + nc;
        if ((e = gemm_f32(t, s)) != hipSuccess) return e;
      }
    }
    if (s1 < d) {  // the super-block's errors to every later column at once
      t.N = d - s1; t.K = s1 - s0;
      t.A = err; t.B = U + s0 * d + s1; t.C = Wp + s1;
      if ((e = gemm_f32(t, s)) != hipSuccess) return e;
    }
  }
  if (rows > 0) {
    const unsigned gx = (unsigned)std::min<int64_t>((d + 1023) / 1024, 64);
    const int vec = (uintptr_t)codes % 4 == 0 && d % 4 == 0;
    hipLaunchKernelGGL(unpermute_kernel, dim3(gx, (unsigned)std::min<int64_t>(rows, 65535)), dim3(256), 0, s, codes_p,
                       rows, d, iperm, codes, vec);
  }
  hipLaunchKernelGGL(loss_kernel, dim3(1), dim3(1024), 0, s, row_loss, rows, loss);
  return hipGetLastError();
}

hipError_t pack(const uint8_t* codes, int64_t rows, int64_t d, int bits, int32_t* packed, hipStream_t s) {
  if (bits > 4) {
    const int64_t n = rows * d;
    if (n <= 0) return hipSuccess;
    const unsigned grid = (unsigned)std::min<int64_t>((n / 16 + 255) / 256 + 1, 65536);
    const int vec = (uintptr_t)codes % 16 == 0 && (uintptr_t)packed % 16 == 0;
    hipLaunchKernelGGL(pack_bytes_kernel, dim3(grid), dim3(256), 0, s, codes, n, reinterpret_cast<uint8_t*>(packed),
                       vec);
    return hipGetLastError();
  }
  const int64_t total = rows * (d / 8);
  if (total <= 0) return hipSuccess;
  const unsigned grid = (unsigned)std::min<int64_t>((total + 255) / 256, 65536);
  const int vec = ((uintptr_t)codes % 8 == 0);
  hipLaunchKernelGGL(pack_kernel, dim3(grid), dim3(256), 0, s, codes, rows, d, packed, vec);
  return hipGetLastError();
}

hipError_t pack_ordered(const uint8_t* codes, int64_t rows, int64_t d, const int32_t* order, int bits, int32_t* packed,
                        hipStream_t s) {
  const int64_t total = rows * (d / (bits <= 4 ? 8 : 4));
  if (total <= 0) return hipSuccess;
  const unsigned grid = (unsigned)std::min<int64_t>((total + 255) / 256, 65536);
  hipLaunchKernelGGL(pack_ordered_kernel, dim3(grid), dim3(256), 0, s, codes, rows, d, order, bits, packed);
  return hipGetLastError();
}

hipError_t permute_columns(const void* in, int64_t m, int64_t d, int64_t ld_in, const int32_t* order, int esz,
                           void* out, int64_t ld_out, hipStream_t s) {
  const int64_t total = m * d;
  if (total <= 0) return hipSuccess;
  const unsigned grid = (unsigned)std::min<int64_t>((total + 255) / 256, 65536);
  hipLaunchKernelGGL(permute_columns_kernel, dim3(grid), dim3(256), 0, s, in, m, d, ld_in, order, esz, out, ld_out);
  return hipGetLastError();
}

hipError_t pack_dense(const uint8_t* codes, int64_t rows, int64_t d, int bits, int32_t* packed, hipStream_t s) {
  const int64_t total = rows * (d * bits / 32);
  if (total <= 0) return hipSuccess;
  const unsigned grid = (unsigned)std::min<int64_t>((total + 255) / 256, 65536);
  hipLaunchKernelGGL(pack_dense_kernel, dim3(grid), dim3(256), 0, s, codes, rows, d, bits, packed);
  return hipGetLastError();
}

}  // namespace gptq
