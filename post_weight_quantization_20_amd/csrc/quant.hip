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

#include <vector>

namespace gptq {
namespace {

struct QArgs {
  float* Wp;             // working weights, processing order, [rows x ldw]
  int64_t ldw;
  int64_t rows, d;
  int64_t s0;            // first column of the super-block
  int sw;                // columns of the super-block
  int B;                 // block width, <= 16 * CPL
  int ldws;              // leading dimension of the super-block's copy in LDS
  const float* U;        // [d x d], processing order
  int64_t g;             // group size (columns)
  int grid_mode;         // 0: groups nest in blocks (g <= B), grids taken inside the column chain;
                         // 1: a group spans blocks of this super-block, its grid taken from the LDS copy
                         //    at its first block; 2: the grid was computed before the launch (a group
                         //    longer than the super-block)
  float maxq;
  uint8_t* codes_p;      // [rows x d], processing order
  float* scales;         // [rows x ngroups]
  int32_t* zeros;        // [rows x ngroups]
  int64_t ngroups;
  int sym;               // symmetric grids
  int compact;           // 16-bit scales, zeros clamped to the code width
  const int32_t* colgrp; // static groups: group of each processing column (its grid is in scales/zeros)
  float* err;            // the super-block's errors: [rows x >= sw] at leading dimension err_ld
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

// One super-block of columns [s0, s0 + sw) for 16 rows of W. The rows' part of the super-block sits
// in LDS for the whole launch. Each block of B columns runs the column chain in registers, and its
// errors then update the super-block's later columns in LDS as 16 x 16 x 4 fp32 MFMA tiles (the lazy
// batch inside the super-block); columns beyond the super-block take the super-block's errors in one
// product after the launch.
// STATIC: every column takes the grid of its static group, colgrp[b + k] (loaded one chunk ahead with
// U's rows); no grid is computed here.
// SUB: the block's chain in 16-column sub-blocks with one column a lane (B a multiple of 16 is not
// needed, but in-block groups must start at multiples of 16 columns): each column's chain updates
// only its own sub-block, and a sub-block's errors reach the block's later columns as 16 x 16 x 4
// MFMA tiles in LDS. Otherwise every lane holds CPL columns of the block and each column's update
// reaches all of them.
template <int CPL, bool STATIC, bool SUB>
__global__ __launch_bounds__(256) void quant_super_kernel(QArgs a) {
  constexpr int BP = 16 * CPL;
  // Row strides of U's block and of the errors, padded so that the MFMA operand reads (four rows of
  // U at once; one error column over the 16 rows) fall in distinct LDS banks.
  constexpr int US = BP + 16, ES = BP + 2;
  extern __shared__ float sm[];
  float* Ws = sm;                  // [16 rows][ldws]: the rows' super-block, updated in place
  float* Us = Ws + 16 * a.ldws;    // [BP][US]: strict upper part of U's block, zeros elsewhere
  float* invd = Us + BP * US;      // [BP]: 1 / U[k][k]
  float* Es = invd + BP;           // [16 rows][ES]: scaled errors of the block
  uint8_t* Qs = reinterpret_cast<uint8_t*>(Es + 16 * ES);  // [16 rows][BP]: codes of the block

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15;
  const int rloc = wave * 4 + (lane >> 4);
  const int64_t row0 = (int64_t)blockIdx.x * 16;
  const int64_t row = row0 + rloc;
  const bool row_ok = row < a.rows;
  const int sw = a.sw;

  // The rows' super-block into LDS; rows past the end read as zeros. Wp's rows are zero-padded to
  // ldw (a multiple of 4), so 16-byte pieces up to the super-block's end rounded to 4 stay inside.
  {
    const bool vec = a.ldw % 4 == 0 && a.s0 % 4 == 0 && (uintptr_t)a.Wp % 16 == 0;
    const int q4 = (sw + 3) / 4;
    for (int e = tid; e < 16 * q4; e += 256) {
      const int r = e / q4, c = (e % q4) * 4;
      const int64_t gr = row0 + r;
      float4 v = float4{0.0f, 0.0f, 0.0f, 0.0f};
      if (gr < a.rows) {
        const float* p = a.Wp + gr * a.ldw + a.s0 + c;
        if (vec) {
          v = *reinterpret_cast<const float4*>(p);
        } else {
          v.x = p[0];
          v.y = c + 1 < sw ? p[1] : 0.0f;
          v.z = c + 2 < sw ? p[2] : 0.0f;
          v.w = c + 3 < sw ? p[3] : 0.0f;
        }
      }
      *reinterpret_cast<float4*>(Ws + r * a.ldws + c) = v;
    }
  }

  float s = 1.0f, z = 0.0f, rs = 1.0f;   // the current group's grid, carried across blocks
  if (!STATIC && a.grid_mode == 2) {
    const int64_t gi = a.s0 / a.g;
    if (row_ok) {
      s = a.scales[row * a.ngroups + gi];
      z = (float)a.zeros[row * a.ngroups + gi];
    }
    rs = 1.0f / s;
  }
  float loss = 0.0f;
  float* wsrow = Ws + rloc * a.ldws;
  const int nblk = (sw + a.B - 1) / a.B;

  for (int jb = 0; jb < nblk; ++jb) {
    const int boff = jb * a.B;            // the block's first column within the super-block
    const int64_t b = a.s0 + boff;        // and within the row
    const int nc = min(a.B, sw - boff);
    __syncthreads();   // the previous block's update of Ws is complete, and Us, Es, Qs are free

    // U's block and its reciprocal diagonal
    bool filled = false;
    if constexpr (CPL >= 4) {
     if (nc == BP && a.d % 4 == 0 && b % 4 == 0 && (uintptr_t)a.U % 16 == 0) {
      // full block: unconditional 16-byte loads, all in flight together
      filled = true;
      constexpr int Q = BP / 4;  // float4 per row
      float4 v[BP * Q / 256];
#pragma unroll
      for (int i = 0; i < BP * Q / 256; ++i) {
        const int e = tid + i * 256, k = e / Q, j = (e % Q) * 4;
        v[i] = *reinterpret_cast<const float4*>(a.U + (b + k) * a.d + b + j);
      }
#pragma unroll
      for (int i = 0; i < BP * Q / 256; ++i) {
        const int e = tid + i * 256, k = e / Q, j = (e % Q) * 4;
        float4 u = v[i];
        u.x = (j + 0 > k) ? u.x : 0.0f;
        u.y = (j + 1 > k) ? u.y : 0.0f;
        u.z = (j + 2 > k) ? u.z : 0.0f;
        u.w = (j + 3 > k) ? u.w : 0.0f;
        *reinterpret_cast<float4*>(Us + k * US + j) = u;
      }
     }
    }
    if (!filled) {
      for (int e = tid; e < BP * BP; e += 256) {
        const int k = e / BP, j = e % BP;
        Us[k * US + j] = (j > k && j < nc) ? a.U[(b + k) * a.d + b + j] : 0.0f;
      }
    }
    for (int k = tid; k < BP; k += 256) invd[k] = (k < nc) ? 1.0f / a.U[(b + k) * a.d + b + k] : 0.0f;

    // lane lr starts with block columns lr*CPL .. lr*CPL+CPL-1 in w[0..CPL-1]
    float w[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) w[c] = (lr * CPL + c < nc) ? wsrow[boff + lr * CPL + c] : 0.0f;

    // a group that spans blocks: its grid from the current weights of its columns in LDS (the
    // earlier blocks' updates of this super-block are in, and those of earlier super-blocks)
    if (!STATIC && a.grid_mode == 1 && b % a.g == 0) {
      const int gend = (int)min<int64_t>(boff + a.g, sw);
      float mn = INFINITY, mx = -INFINITY;
      for (int c = boff + lr; c < gend; c += 16) {
        const float v = wsrow[c];
        mn = fminf(mn, v);
        mx = fmaxf(mx, v);
      }
      mn = fminf(mn, row_ror<8>(mn)); mx = fmaxf(mx, row_ror<8>(mx));
      mn = fminf(mn, row_ror<4>(mn)); mx = fmaxf(mx, row_ror<4>(mx));
      mn = fminf(mn, row_ror<2>(mn)); mx = fmaxf(mx, row_ror<2>(mx));
      mn = fminf(mn, row_ror<1>(mn)); mx = fmaxf(mx, row_ror<1>(mx));
      make_grid(mn, mx, a.maxq, a.sym != 0, a.compact != 0, s, z, rs);
      if (lr == 0 && row_ok) {
        const int64_t gi = (uint32_t)b / (uint32_t)a.g;   // column and group indices stay below 2^31
        a.scales[row * a.ngroups + gi] = s;
        a.zeros[row * a.ngroups + gi] = (int32_t)z;
      }
    }
    __syncthreads();   // U's block staged

    if constexpr (SUB) {
      const int l16 = lane & 15, lq = lane >> 4;
      float* esrow = Es + rloc * ES;
      uint8_t* qsrow = Qs + rloc * BP;
      for (int cs = 0; cs < nc; cs += 16) {
        const int ncs = min(16, nc - cs);
        float ws = (lr < ncs) ? wsrow[boff + cs + lr] : 0.0f;   // this lane's column
        // U[cs + c][cs + lr] / U[cs + c][cs + c], zero unless lr > c: the update of this lane's column
        // by column c's unscaled difference w - s (q - z), scaled here, off the chain
        float u[16];
#pragma unroll
        for (int c = 0; c < 16; ++c) u[c] = Us[(cs + c) * US + cs + lr] * invd[cs + c];
        // a group starting here (in-block groups of a multiple of 16 columns): its grid from the
        // current weights of its columns, which every earlier sub-block's errors have reached
        if (!STATIC && a.grid_mode == 0 && cs % a.g == 0) {
          const int gend = (int)min<int64_t>(cs + a.g, nc);
          float mn = INFINITY, mx = -INFINITY;
          for (int c = cs + lr; c < gend; c += 16) {
            const float v = wsrow[boff + c];
            mn = fminf(mn, v);
            mx = fmaxf(mx, v);
          }
          mn = fminf(mn, row_ror<8>(mn)); mx = fmaxf(mx, row_ror<8>(mx));
          mn = fminf(mn, row_ror<4>(mn)); mx = fmaxf(mx, row_ror<4>(mx));
          mn = fminf(mn, row_ror<2>(mn)); mx = fmaxf(mx, row_ror<2>(mx));
          mn = fminf(mn, row_ror<1>(mn)); mx = fmaxf(mx, row_ror<1>(mx));
          make_grid(mn, mx, a.maxq, a.sym != 0, a.compact != 0, s, z, rs);
          if (lr == 0 && row_ok) {
            const int64_t gi = (uint32_t)(b + cs) / (uint32_t)a.g;
            a.scales[row * a.ngroups + gi] = s;
            a.zeros[row * a.ngroups + gi] = (int32_t)z;
          }
        }
        // static groups: this lane's column's grid, broadcast to the row at each column
        float sg = 1.0f, zg = 0.0f, rsg = 1.0f;
        if constexpr (STATIC) {
          const int64_t G = a.colgrp[b + cs + min(lr, ncs - 1)];
          if (row_ok) {
            sg = a.scales[row * a.ngroups + G];
            zg = (float)a.zeros[row * a.ngroups + G];
          }
          rsg = 1.0f / sg;
        }
        // Column c: every lane of the row runs the chain on the broadcast weight, and the lanes that
        // hold later columns of the sub-block take its update, the difference w - s (q - z) times
        // U's row scaled by 1 / U[c][c] (zero for lanes lr <= c). Columns past the block's end hold
        // zeros with zero rows of U and 1 / U[k][k] = 0, so they change nothing.
        static_for<0, 16>([&](auto cc) {
          constexpr int c = decltype(cc)::value;
          if constexpr (STATIC) {
            s = row_bcast<c>(sg);
            z = row_bcast<c>(zg);
            rs = row_bcast<c>(rsg);
          }
          const float wk = row_bcast<c>(ws);
          const float x = div_rn(wk, s, rs);
          const float qd = __builtin_amdgcn_fmed3f(rintf(x), -z, a.maxq - z);
          ws = __builtin_fmaf(-__builtin_fmaf(-s, qd, wk), u[c], ws);
        });
        // After column lr, nothing changes lane lr's weight again: it is the weight its column was
        // quantized from, and the same steps give that column's code and error once more, here.
        {
          const float so = STATIC ? sg : s, zo = STATIC ? zg : z, rso = STATIC ? rsg : rs;
          const float x = div_rn(ws, so, rso);
          const float qd = __builtin_amdgcn_fmed3f(rintf(x), -zo, a.maxq - zo);
          float e = __builtin_fmaf(-so, qd, ws) * invd[cs + lr];
          e = lr < ncs ? e : 0.0f;
          loss = __builtin_fmaf(e, e, loss);
          esrow[cs + lr] = e;
          qsrow[cs + lr] = (uint8_t)(qd + zo);
        }
        // ... into the block's later columns, for this wave's four rows only, so no other wave waits:
        // v_mfma_f32_4x4x1f32 with 16 blocks takes A[l % 4][k] (the same four rows in every block)
        // and B[k][l] from lane l, and register r of lane l holds row r, column l, of a 4 x 64 tile.
        // A = E (the wave's rows by the sub-block's columns), B = U's rows of the sub-block, C = 64
        // of the block's later columns of Ws. The lanes' stores above and the reads below cross
        // lanes of this wave only.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_wave_barrier();
        const int c0 = cs + 16;
        if (c0 < nc) {
          const int rb = 4 * wave;   // the wave's first row of the 16
          float av[16];
#pragma unroll
          for (int k = 0; k < 16; ++k) av[k] = -Es[(rb + (lane & 3)) * ES + cs + k];
          // columns c0 + lane and c0 + 64 + lane; each sum split over even and odd k, so that four
          // independent accumulators hide the MFMA latency
          const bool two = nc - c0 > 64;
          int cr[2];
          bool ok[2];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int col = c0 + 64 * h + lane;
            ok[h] = col < nc && (h == 0 || two);
            cr[h] = ok[h] ? col : cs;   // a column inside U's block for the loads
          }
          floatx4 acc[2][2];
          float bv[2][16];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            if (h == 1 && !two) break;
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[h][0][r] = Ws[(rb + r) * a.ldws + boff + cr[h]];
            acc[h][1] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int k = 0; k < 16; ++k) bv[h][k] = Us[(cs + k) * US + cr[h]];
          }
          if (two) {
#pragma unroll
            for (int k = 0; k < 16; ++k) {
              acc[0][k & 1] = __builtin_amdgcn_mfma_f32_4x4x1f32(av[k], bv[0][k], acc[0][k & 1], 0, 0, 0);
              acc[1][k & 1] = __builtin_amdgcn_mfma_f32_4x4x1f32(av[k], bv[1][k], acc[1][k & 1], 0, 0, 0);
            }
          } else {
#pragma unroll
            for (int k = 0; k < 16; ++k)
              acc[0][k & 1] = __builtin_amdgcn_mfma_f32_4x4x1f32(av[k], bv[0][k], acc[0][k & 1], 0, 0, 0);
          }
#pragma unroll
          for (int h = 0; h < 2; ++h)
            if (ok[h]) {
#pragma unroll
              for (int r = 0; r < 4; ++r) Ws[(rb + r) * a.ldws + boff + c0 + 64 * h + lane] = acc[h][0][r] + acc[h][1][r];
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_wave_barrier();   // this wave's Ws columns updated before its next sub-block
      }
      __syncthreads();   // the block's codes and errors of all 16 rows are in Qs and Es
    } else {
    // groups nest inside blocks when g <= B, so they start at block columns 0, g, 2g, ...
    int next_group = (!STATIC && a.grid_mode == 0) ? 0 : (1 << 30);
    const int gsz = (int)min<int64_t>(a.g, (int64_t)BP);

    // Chunk o quantizes block columns o*CPL .. o*CPL+CPL-1. Before it, the lanes of each row have
    // been rotated o times by one lane, so lane 0 holds those columns and lane l holds the columns
    // of original lane (l + o) mod 16 (already quantized ones meet zeros in U and stay unchanged).
    // What a chunk reads from LDS (U's rows for its columns, their reciprocal diagonal) is read one
    // chunk ahead, into the other of two register sets; U and the diagonal are not written during the
    // chain, and the chunk's own stores go to the codes and errors.
    const int nchunks = (nc + CPL - 1) / CPL;
    // static groups: the scale and zero of each of a chunk's columns (one chunk ahead, like U's rows)
    float sA[STATIC ? CPL : 1], zA[STATIC ? CPL : 1], sB[STATIC ? CPL : 1], zB[STATIC ? CPL : 1];
    auto fetch_grid = [&](int o, float (&sv)[STATIC ? CPL : 1], float (&zv)[STATIC ? CPL : 1]) {
      if constexpr (STATIC) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const int k = min(o * CPL + c, nc - 1);
          const int64_t G = a.colgrp[b + k];
          sv[c] = row_ok ? a.scales[row * a.ngroups + G] : 1.0f;
          zv[c] = row_ok ? (float)a.zeros[row * a.ngroups + G] : 0.0f;
        }
      }
    };
    auto fetch = [&](int o, float (&iv)[CPL], float (&ur)[CPL][CPL]) {
      const int cbase = ((lr + o) & 15) * CPL;
      lds_load<CPL>(invd + o * CPL, iv);
#pragma unroll
      for (int c = 0; c < CPL; ++c) lds_load<CPL>(Us + (o * CPL + c) * US + cbase, ur[c]);
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
            const int64_t gi = (uint32_t)(b + k) / (uint32_t)a.g;
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
          Es[rloc * ES + o * CPL + c] = ev[c];
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
    // the errors of columns nc .. 16 ceil(nc / 16) - 1 read as zeros in the update below
    for (int e = tid; e < 16 * 16; e += 256) {
      const int k = nc + e % 16;
      if (k < (nc + 15) / 16 * 16) Es[(e / 16) * ES + k] = 0.0f;
    }
    __syncthreads();   // the block's codes and errors are in Qs and Es
    }

    if (row_ok) {
      uint8_t* crow = a.codes_p + row * a.d + b;
      float* erow = a.err + row * a.err_ld + boff;
      const int j0 = lr * CPL;
      const bool vec = CPL == 8 && nc == BP && a.d % 8 == 0 && b % 8 == 0 && a.err_ld % 4 == 0 && boff % 4 == 0 &&
                       (uintptr_t)a.codes_p % 8 == 0 && (uintptr_t)a.err % 16 == 0;
      if constexpr (CPL == 8) {
        if (vec) {
          *reinterpret_cast<uint2*>(crow + j0) = *reinterpret_cast<const uint2*>(Qs + rloc * BP + j0);
          const float2* es = reinterpret_cast<const float2*>(Es + rloc * ES + j0);   // rows 8-byte aligned
          const float2 e0 = es[0], e1 = es[1], e2 = es[2], e3 = es[3];
          *reinterpret_cast<float4*>(erow + j0) = float4{e0.x, e0.y, e1.x, e1.y};
          *reinterpret_cast<float4*>(erow + j0 + 4) = float4{e2.x, e2.y, e3.x, e3.y};
        }
      }
      if (!(CPL == 8 && vec)) {
#pragma unroll
        for (int t = 0; t < CPL; ++t) {
          const int j = j0 + t;
          if (j < nc) {
            crow[j] = Qs[rloc * BP + j];
            erow[j] = Es[rloc * ES + j];
          }
        }
      }
    }

    // The block's errors into the super-block's later columns: Ws[:, c0:sw] -= E U[b:b+nc, s0+c0:s0+sw].
    // v_mfma_f32_16x16x4f32 takes A[l % 16][k + l / 16] and B[k + l / 16][l % 16] from lane l, and
    // register r of its result holds row 4 (l / 16) + r, column l % 16: here A = E (the 16 rows by the
    // block's columns), B = U's rows of the block, C = Ws. The columns go in 32-column strips, each two
    // 16-column tiles interleaved: tile u of strip j gives its column n to global column
    // c0 + 32 j + 2 n + u, so that one 8-byte load fetches a lane's operands of both tiles. Wave w
    // holds strips w, w + 4, ... (up to MS at once) with every accumulator live, and the loop runs over
    // k outermost, the operands of the next KC k-steps in flight while the current ones feed the MFMAs.
    const int c0 = boff + nc;
    if (c0 < sw) {
      const int l16 = lane & 15, lq = lane >> 4;
      const int ksteps = (nc + 3) / 4;
      const int nst = (sw - c0 + 31) / 32;
      constexpr int MS = 3, KC = 4;
      // 8-byte loads when aligned and both columns of every pair exist together (an even width left)
      const bool v2 = (a.s0 + c0) % 2 == 0 && a.d % 2 == 0 && (uintptr_t)a.U % 8 == 0 && (sw - c0) % 2 == 0;
      auto strips = [&](auto vec) {
        constexpr bool V2 = decltype(vec)::value;
        for (int j0 = 0; j0 < nst; j0 += 4 * MS) {
          // Strip m's columns of this lane (within the super-block), and the columns its loads read:
          // a column past the super-block reads column c0 instead, into an accumulator that is not
          // stored. The loads are unconditional: a masked load, or a select on its value, would
          // make the wave wait for it ahead of the MFMAs that do not need it.
          int col[MS], rd0[MS], rd1[MS];
          bool okc[MS][2];
          floatx4 acc[MS][2];
#pragma unroll
          for (int m = 0; m < MS; ++m) {
            const int j = j0 + wave + 4 * m;
            col[m] = c0 + 32 * j + 2 * l16;
            okc[m][0] = j < nst && col[m] < sw;
            okc[m][1] = j < nst && col[m] + 1 < sw;
            rd0[m] = okc[m][0] ? col[m] : c0;
            rd1[m] = okc[m][1] ? col[m] + 1 : c0;
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
              for (int r = 0; r < 4; ++r)
                acc[m][u][r] = okc[m][u] ? Ws[(4 * lq + r) * a.ldws + col[m] + u] : 0.0f;
          }
          float avA[KC], avB[KC];
          float2 bvA[KC][MS], bvB[KC][MS];
          // The errors of columns nc .. 16 ceil(nc / 16) - 1 are zero, which covers every k the
          // k-steps reach past the block; those k read U's row b.
          auto fetch = [&](int kg, float (&av)[KC], float2 (&bv)[KC][MS]) {
#pragma unroll
            for (int i = 0; i < KC; ++i) {
              const int k = 4 * (kg + i) + lq;
              av[i] = -Es[l16 * ES + k];
              const float* ur = a.U + (b + (k < nc ? k : 0)) * a.d + a.s0;
#pragma unroll
              for (int m = 0; m < MS; ++m) {
                if constexpr (V2) bv[i][m] = *reinterpret_cast<const float2*>(ur + rd0[m]);
                else bv[i][m] = float2{ur[rd0[m]], ur[rd1[m]]};
              }
            }
          };
          auto mma = [&](const float (&av)[KC], const float2 (&bv)[KC][MS]) {
#pragma unroll
            for (int i = 0; i < KC; ++i)
#pragma unroll
              for (int m = 0; m < MS; ++m) {
                acc[m][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[i], bv[i][m].x, acc[m][0], 0, 0, 0);
                acc[m][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[i], bv[i][m].y, acc[m][1], 0, 0, 0);
              }
          };
          fetch(0, avA, bvA);
          for (int kg = 0; kg < ksteps; kg += 2 * KC) {
            if (kg + KC < ksteps) fetch(kg + KC, avB, bvB);
            mma(avA, bvA);
            if (kg + KC < ksteps) {
              if (kg + 2 * KC < ksteps) fetch(kg + 2 * KC, avA, bvA);
              mma(avB, bvB);
            }
          }
#pragma unroll
          for (int m = 0; m < MS; ++m)
#pragma unroll
            for (int u = 0; u < 2; ++u)
              if (okc[m][u]) {
#pragma unroll
                for (int r = 0; r < 4; ++r) Ws[(4 * lq + r) * a.ldws + col[m] + u] = acc[m][u][r];
              }
        }
      };
      if (v2) strips(std::true_type{});
      else strips(std::false_type{});
    }
  }
  if constexpr (SUB) {
    // each lane summed its own columns' squared errors: the row's sum over its 16 lanes
    loss += row_ror<8>(loss);
    loss += row_ror<4>(loss);
    loss += row_ror<2>(loss);
    loss += row_ror<1>(loss);
  }
  if (lr == 0 && row_ok) a.row_loss[row] += (double)loss;
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
// multiple of 4). A thread writes four consecutive columns, as one 16-byte store when Wp allows. With
// pvec (perm 16-byte aligned, W's rows starting on 4-element boundaries of an aligned base), a thread
// reads its four entries of perm at once, and where they are four consecutive columns it reads their
// weights with one 8-byte (fp16, bf16) or 16-byte (fp32) load.
__global__ __launch_bounds__(256) void gather_w_kernel(const void* __restrict__ W, int dtype, int64_t ldw_in,
                                                       int64_t rows, int64_t d, const int32_t* __restrict__ perm,
                                                       float* __restrict__ Wp, int64_t ldw, int vec, int pvec) {
  for (int64_t r = blockIdx.y; r < rows; r += gridDim.y)
    for (int64_t j = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4; j < ldw; j += (int64_t)gridDim.x * 1024) {
      float v[4];
      bool done = false;
      if (pvec && j + 4 <= d) {
        const int4 pj = *reinterpret_cast<const int4*>(perm + j);
        const int64_t e = r * ldw_in + pj.x;
        if (pj.y == pj.x + 1 && pj.z == pj.x + 2 && pj.w == pj.x + 3 && e % 4 == 0) {
          if (dtype == F32) {
            const float4 q = *reinterpret_cast<const float4*>(static_cast<const float*>(W) + e);
            v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
          } else {
            const uint2 q = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(W) + e);
            const uint16_t h[4] = {(uint16_t)(q.x & 0xffffu), (uint16_t)(q.x >> 16), (uint16_t)(q.y & 0xffffu),
                                   (uint16_t)(q.y >> 16)};
#pragma unroll
            for (int t = 0; t < 4; ++t) v[t] = dtype == F16 ? (float)__builtin_bit_cast(_Float16, h[t]) : bf16_bits_to_f32(h[t]);
          }
        } else {
          const int pp[4] = {pj.x, pj.y, pj.z, pj.w};
#pragma unroll
          for (int t = 0; t < 4; ++t) v[t] = load_as_f32(W, dtype, r * ldw_in + pp[t]);
        }
        done = true;
      }
      if (!done) {
#pragma unroll
        for (int t = 0; t < 4; ++t) v[t] = (j + t < d) ? load_as_f32(W, dtype, r * ldw_in + perm[j + t]) : 0.0f;
      }
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
// consecutive codes. With vec (rows of 4-byte multiples, codes and codes_p 4-byte aligned, iperm
// 16-byte aligned) it reads four entries of iperm at once, reads the codes with one 4-byte load where
// they are four consecutive positions starting on a 4-byte boundary, and stores them as one word.
__global__ __launch_bounds__(256) void unpermute_kernel(const uint8_t* __restrict__ codes_p, int64_t rows, int64_t d,
                                                        const int32_t* __restrict__ iperm, uint8_t* __restrict__ codes,
                                                        int vec) {
  for (int64_t r = blockIdx.y; r < rows; r += gridDim.y)
    for (int64_t c = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4; c < d; c += (int64_t)gridDim.x * 1024) {
      const uint8_t* src = codes_p + r * d;
      uint8_t* dst = codes + r * d + c;
      if (vec && c + 4 <= d) {
        const int4 ic = *reinterpret_cast<const int4*>(iperm + c);
        uint32_t w;
        if (ic.y == ic.x + 1 && ic.z == ic.x + 2 && ic.w == ic.x + 3 && (r * d + ic.x) % 4 == 0)
          w = *reinterpret_cast<const uint32_t*>(src + ic.x);
        else
          w = src[ic.x] | (src[ic.y] << 8) | (src[ic.z] << 16) | ((uint32_t)src[ic.w] << 24);
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

int64_t super_width_max(int B) { return std::max<int64_t>(1, 512 / B) * B; }

// LDS leading dimension of a super-block's copy: whole 16-column tiles plus 4 floats of padding.
int super_ld(int sw) { return (sw + 15) / 16 * 16 + 4; }

template <int CPL>
size_t qsmem(int sw) {
  constexpr size_t BP = 16 * CPL;
  return (16 * (size_t)super_ld(sw) + BP * (BP + 16) + BP + 16 * (BP + 2)) * sizeof(float) + 16 * BP;
}

template <int CPL, bool STATIC, bool SUB>
void launch_super(const QArgs& a, hipStream_t s) {
  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute((const void*)quant_super_kernel<CPL, STATIC, SUB>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)qsmem<CPL>(512 + 16 * CPL));
    attr = true;
  }
  hipLaunchKernelGGL((quant_super_kernel<CPL, STATIC, SUB>), dim3((unsigned)((a.rows + 15) / 16)), dim3(256),
                     qsmem<CPL>(a.sw), s, a);
}

template <int CPL>
void launch_super(const QArgs& a, bool is_static, hipStream_t s) {
  if (is_static) launch_super<CPL, true, false>(a, s);
  else launch_super<CPL, false, false>(a, s);
}

// The sub-block chain for 128-column blocks (B > 64), when in-block groups start at multiples of 16.
void launch_super_sub(const QArgs& a, bool is_static, hipStream_t s) {
  if (is_static) launch_super<8, true, true>(a, s);
  else launch_super<8, false, true>(a, s);
}

int cpl_for(int B) { return B <= 16 ? 1 : B <= 32 ? 2 : B <= 64 ? 4 : 8; }

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
                    hipStream_t s, double* part_ms) {
  const QuantLayout L = quant_layout(rows, d, B);
  // measurement: an event after each group of launches, the interval before it charged to a part
  std::vector<hipEvent_t> evs;
  std::vector<int> parts;
  auto mark = [&](int part) {
    if (!part_ms) return;
    hipEvent_t ev = nullptr;
    if (hipEventCreate(&ev) != hipSuccess) return;
    if (hipEventRecord(ev, s) != hipSuccess) {
      (void)hipEventDestroy(ev);
      return;
    }
    evs.push_back(ev);
    parts.push_back(part);
  };
  mark(2);
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
    const int esz = w_dtype == F32 ? 4 : 2;
    const int pvec = (uintptr_t)perm % 16 == 0 && (uintptr_t)W % (4 * esz) == 0;
    hipLaunchKernelGGL(gather_w_kernel, dim3(gx, (unsigned)std::min<int64_t>(rows, 65535)), dim3(256), 0, s, W, w_dtype,
                       ld_w, rows, d, perm, Wp, L.ldw, vec, pvec);
    hipLaunchKernelGGL(zero_f64, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s, row_loss, rows);
  }
  mark(2);
  hipError_t e;
  const int cpl = cpl_for(B);
  const int64_t sw = super_width(B, g, d);
  // where group grids are taken (see QArgs::grid_mode)
  const int grid_mode = static_groups ? 2 : g <= B ? 0 : g <= sw ? 1 : 2;
  GemmArgs t{};  // W[:, s1:] -= Err U[s0:s1, s1:]
  t.M = rows; t.transA = 0; t.ldb = d; t.transB = 0; t.ldc = L.ldw;
  t.alpha = -1.0f; t.beta = 1.0f; t.tri = 0; t.lda = L.ld_err;
  for (int64_t s0 = 0; s0 < d && rows > 0; s0 += sw) {
    const int64_t s1 = std::min(d, s0 + sw);
    if (!static_groups && grid_mode == 2 && s0 % g == 0) {
      // a group longer than the super-block: its grid from the current weights of all its columns
      hipLaunchKernelGGL(group_grid_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, Wp, L.ldw, rows, s0,
                         std::min<int64_t>(g, d - s0), maxq, sym, compact, s0 / g, scales, zeros, ngroups);
    }
    QArgs a;
    a.Wp = Wp; a.ldw = L.ldw; a.rows = rows; a.d = d; a.s0 = s0; a.sw = (int)(s1 - s0); a.B = B;
    a.ldws = super_ld(a.sw); a.U = U; a.g = g; a.grid_mode = grid_mode; a.maxq = maxq; a.codes_p = codes_p;
    a.scales = scales; a.zeros = zeros; a.ngroups = ngroups; a.err = err; a.err_ld = L.ld_err;
    a.row_loss = row_loss; a.sym = sym; a.compact = compact; a.colgrp = colgrp;
    const bool st = static_groups != 0;
    const bool sub = cpl == 8 && (st || grid_mode != 0 || g % 16 == 0);
    if (sub) {
      launch_super_sub(a, st, s);
    } else {
      switch (cpl) {
        case 1: launch_super<1>(a, st, s); break;
        case 2: launch_super<2>(a, st, s); break;
        case 4: launch_super<4>(a, st, s); break;
        default: launch_super<8>(a, st, s); break;
      }
    }
    mark(0);
    if (s1 < d) {  // the super-block's errors to every later column at once
      t.N = d - s1; t.K = s1 - s0;
      t.A = err; t.B = U + s0 * d + s1; t.C = Wp + s1;
      if ((e = gemm_f32(t, s)) != hipSuccess) return e;
      mark(1);
    }
  }
  if (rows > 0) {
    const unsigned gx = (unsigned)std::min<int64_t>((d + 1023) / 1024, 64);
    const int vec = (uintptr_t)codes % 4 == 0 && d % 4 == 0 && (uintptr_t)iperm % 16 == 0 && (uintptr_t)codes_p % 4 == 0;
    hipLaunchKernelGGL(unpermute_kernel, dim3(gx, (unsigned)std::min<int64_t>(rows, 65535)), dim3(256), 0, s, codes_p,
                       rows, d, iperm, codes, vec);
  }
  hipLaunchKernelGGL(loss_kernel, dim3(1), dim3(1024), 0, s, row_loss, rows, loss);
  e = hipGetLastError();
  if (part_ms) {
    mark(2);
    part_ms[0] = part_ms[1] = part_ms[2] = 0.0;
    if (e == hipSuccess && !evs.empty()) e = hipEventSynchronize(evs.back());
    for (size_t i = 1; i < evs.size() && e == hipSuccess; ++i) {
      float ms = 0.0f;
      if ((e = hipEventElapsedTime(&ms, evs[i - 1], evs[i])) == hipSuccess) part_ms[parts[i]] += ms;
    }
    for (hipEvent_t ev : evs) (void)hipEventDestroy(ev);
  }
  return e;
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
