// Hessian accumulation H += 2 X^T X for fp16 / bf16 activations on CDNA4 matrix cores.
//
// The layer Hessian is proportional to the product of the calibration inputs with their transpose
// and is shared by every row of W (GPTQ tools page, "How it works", Step 3; the sketch forms
// 2 X^T X / n, and the normalisation by n happens when the Hessian is damped).
//
// X arrives token-major ([tokens x d], features contiguous) and the product contracts over tokens,
// so both MFMA operands need 8 consecutive tokens of one feature per lane. Each thread loads an
// 8-token x 8-feature block with eight 16-byte loads, transposes it in registers and stores eight
// 16-byte rows into a feature-major LDS tile (double buffered: the next stage's stores overlap the
// current stage's MFMAs, one barrier per stage). A 256-thread workgroup (4 wave64s, 2x2) owns a
// 256x256 tile of H in the upper triangle; each wave owns 128x128 (4x4 blocks of
// v_mfma_f32_32x32x16_{f16,bf16}, 256 accumulators per lane), which needs half the LDS reads per
// MFMA of a 64x128 wave tile. Products of fp16/bf16 values are exact in fp32; accumulation is fp32.
//
// When the upper-triangle tiles alone cannot fill the 256 CUs, the token range is split S ways.
// Each split writes its partial tile to the workspace, and the last split to finish a tile (an
// agent-scope atomic counter) adds the partials to H in split order, so the result does not
// depend on scheduling.
#include "common.hpp"

#include <cmath>

namespace gptq {
namespace {

constexpr int HT = 256;            // tile edge (features)
constexpr int HK = 64;             // tokens per LDS stage
constexpr int HROW = HK + 8;       // LDS row length in halves (16-byte pad)
constexpr int NCU = 256;

struct HessArgs {
  float* H;
  int64_t d;
  const uint16_t* X;   // fp16 or bf16 bit patterns
  int64_t n, ldx;
  int T;               // tiles per dimension
  int ntiles;          // T (T + 1) / 2
  int S;               // token splits: 1, or a multiple of 8 (split s runs on XCD s % 8)
  int per_xcd;         // S == 1: tiles per XCD (contiguous in the tile order)
  int64_t split_len;   // tokens per split (multiple of HK)
  float* partial;      // [ntiles * S][HT * HT] when S > 1
  int* counters;       // [ntiles] when S > 1
  int vec;             // 16-byte loads allowed
};

// Upper-triangle tile pairs (ti <= tj) in an order that keeps neighbours close: super-blocks of
// G x G tiles in row order of the upper triangle of super-blocks, row order inside each. Workgroups
// that run together on one XCD take consecutive slots, so they share few feature blocks of X and
// reuse them from that XCD's L2.
constexpr int G = 8;

GPTQ_DEV void tile_at(int slot, int T, int& ti, int& tj) {
  const int NSB = (T + G - 1) / G;
  for (int R = 0; R < NSB; ++R) {
    const int r0 = R * G, r1 = min(T, r0 + G);
    for (int C = R; C < NSB; ++C) {
      const int c0 = C * G, c1 = min(T, c0 + G);
      for (int r = r0; r < r1; ++r) {
        const int cs = max(c0, r);
        const int cnt = max(0, c1 - cs);
        if (slot < cnt) { ti = r; tj = cs + slot; return; }
        slot -= cnt;
      }
    }
  }
  ti = tj = 0;
}

// Loads an 8-token x 8-feature block starting at (tok, f) into 8 registers of 8 halves.
GPTQ_DEV void load_block(const HessArgs& a, int64_t tok, int64_t tok_end, int64_t f, u32x4 (&r)[8]) {
  if (a.vec && tok + 8 <= tok_end && f + 8 <= a.d) {
    // whole block in range: eight unconditional 16-byte loads in flight together
    const uint16_t* p = a.X + tok * a.ldx + f;
#pragma unroll
    for (int t = 0; t < 8; ++t) r[t] = *reinterpret_cast<const u32x4*>(p + t * a.ldx);
    return;
  }
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int64_t tt = tok + t;
    const uint16_t* p = a.X + tt * a.ldx + f;
    if (a.vec && tt < tok_end && f + 7 < a.d) {
      r[t] = *reinterpret_cast<const u32x4*>(p);
    } else {
      uint32_t h[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) h[e] = (tt < tok_end && f + e < a.d) ? p[e] : 0u;
      r[t] = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
    }
  }
}

// Transposes the block (r[t] holds features 0..7 of token t) and stores feature rows of 8 tokens.
GPTQ_DEV void store_block(uint16_t* tile, int fl, int tl, const u32x4 (&r)[8]) {
#pragma unroll
  for (int ff = 0; ff < 8; ++ff) {
    uint32_t w[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t x = r[2 * p][ff >> 1], y = r[2 * p + 1][ff >> 1];
      w[p] = (ff & 1) ? ((x >> 16) | (y & 0xffff0000u)) : ((x & 0xffffu) | (y << 16));
    }
    *reinterpret_cast<u32x4*>(tile + (fl + ff) * HROW + tl) = u32x4{w[0], w[1], w[2], w[3]};
  }
}

template <typename V>
GPTQ_DEV floatx16 mfma16(V a, V b, floatx16 c);
template <>
GPTQ_DEV floatx16 mfma16<half8>(half8 a, half8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
template <>
GPTQ_DEV floatx16 mfma16<bf16x8>(bf16x8 a, bf16x8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <typename V>
__global__ __launch_bounds__(256) void hess_kernel(HessArgs a) {
  extern __shared__ __align__(16) uint16_t smem[];
  constexpr int TILE = HT * HROW;   // halves per operand tile
  // buffers: [stage][operand] -> smem + (2 * stage + operand) * TILE

  // Workgroup b runs on XCD b % 8. With token splits, XCD x takes splits x, x + 8, ... and walks
  // every tile for each; without, it takes a contiguous run of tiles over all tokens.
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  int tile, split;
  if (a.S > 1) {
    tile = slot % a.ntiles;
    split = xcd + 8 * (slot / a.ntiles);
  } else {
    tile = xcd * a.per_xcd + slot;
    split = 0;
    if (slot >= a.per_xcd || tile >= a.ntiles) return;
  }
  int ti, tj;
  tile_at(tile, a.T, ti, tj);
  const bool diag = ti == tj;
  const int64_t fa = (int64_t)ti * HT, fb = (int64_t)tj * HT;
  const int64_t t_begin = (int64_t)split * a.split_len;
  const int64_t t_end = min(a.n, t_begin + a.split_len);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int li = lane & 31, lk = lane >> 5;

  // loader: each thread moves one 8-token x 8-feature block of each operand per stage; 8
  // consecutive lanes take 8 token blocks of one feature block (128-byte global segments,
  // conflict-free 16-byte LDS row stores)
  const int fl = (tid >> 3) * 8, tl = (tid & 7) * 8;

  floatx16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  u32x4 ra[8], rb[8];
  int64_t t0 = t_begin;
  int buf = 0;
  if (t0 < t_end) {
    load_block(a, t0 + tl, t_end, fa + fl, ra);
    if (!diag) load_block(a, t0 + tl, t_end, fb + fl, rb);
    store_block(smem, fl, tl, ra);
    if (!diag) store_block(smem + TILE, fl, tl, rb);
  }
  __syncthreads();
  for (; t0 < t_end; t0 += HK) {
    const bool more = t0 + HK < t_end;
    if (more) {
      load_block(a, t0 + HK + tl, t_end, fa + fl, ra);
      if (!diag) load_block(a, t0 + HK + tl, t_end, fb + fl, rb);
    }
    const uint16_t* Xa = smem + (2 * buf) * TILE;
    const uint16_t* Xb = diag ? Xa : Xa + TILE;
    // operands of the next 16 tokens are read from LDS while the MFMAs of the current 16 run
    V av[2][4], bv[2][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      av[0][i] = *reinterpret_cast<const V*>(Xa + (wm * 128 + i * 32 + li) * HROW + 8 * lk);
      bv[0][i] = *reinterpret_cast<const V*>(Xb + (wn * 128 + i * 32 + li) * HROW + 8 * lk);
    }
#pragma unroll
    for (int s4 = 0; s4 < HK / 16; ++s4) {
      const int c = s4 & 1, n = c ^ 1;
      if (s4 + 1 < HK / 16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          av[n][i] = *reinterpret_cast<const V*>(Xa + (wm * 128 + i * 32 + li) * HROW + (s4 + 1) * 16 + 8 * lk);
          bv[n][i] = *reinterpret_cast<const V*>(Xb + (wn * 128 + i * 32 + li) * HROW + (s4 + 1) * 16 + 8 * lk);
        }
      }
      // keep the reads above ahead of this step's MFMAs (the scheduler would sink them)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16<V>(av[c][i], bv[c][j], acc[i][j]);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (more) {
      uint16_t* nb = smem + (2 * (buf ^ 1)) * TILE;
      store_block(nb, fl, tl, ra);
      if (!diag) store_block(nb + TILE, fl, tl, rb);
    }
    __syncthreads();
    buf ^= 1;
  }

  // Epilogue: accumulator register r of lane l holds row 8*(r/4) + 4*(l/32) + r%4, column l%32.
  if (a.S == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t m = fa + wm * 128 + i * 32 + 8 * (r >> 2) + 4 * lk + (r & 3);
          const int64_t c = fb + wn * 128 + j * 32 + li;
          if (m < a.d && c < a.d) {
            float* h = a.H + m * a.d + c;
            *h = __builtin_fmaf(2.0f, acc[i][j][r], *h);
          }
        }
    return;
  }

  float* part = a.partial + ((int64_t)tile * a.S + split) * (HT * HT);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = wm * 128 + i * 32 + 8 * (r >> 2) + 4 * lk + (r & 3);
        const int c = wn * 128 + j * 32 + li;
        part[m * HT + c] = acc[i][j][r];
      }
  __threadfence();
  __syncthreads();
  __shared__ int last;
  if (tid == 0) {
    const int prev = __hip_atomic_fetch_add(a.counters + tile, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    last = (prev == a.S - 1);
  }
  __syncthreads();
  if (!last) return;
  __threadfence();
  const float* base = a.partial + (int64_t)tile * a.S * (HT * HT);
  for (int e = tid * 4; e < HT * HT; e += 256 * 4) {
    floatx4 s = *reinterpret_cast<const floatx4*>(base + e);
    for (int q = 1; q < a.S; ++q) s += *reinterpret_cast<const floatx4*>(base + (int64_t)q * HT * HT + e);
    const int m = e / HT, c = e % HT;
    const int64_t gm = fa + m;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t gc = fb + c + k;
      if (gm < a.d && gc < a.d) {
        float* h = a.H + gm * a.d + gc;
        *h = __builtin_fmaf(2.0f, s[k], *h);
      }
    }
  }
}

__global__ void zero_ints(int* p, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// Token splits: none when the tiles alone give every CU several workgroups; otherwise 8 (one per
// XCD), or a larger multiple of 8 when the last round would be less than 80% full, as long as
// each split keeps 16 stages.
int choose_splits(int64_t ntiles, int64_t n) {
  if (ntiles >= 3 * NCU) return 1;
  if (n < 8 * 16 * HK) return 1;
  for (int s = 8; s <= 32 && n >= (int64_t)s * 16 * HK; s += 8) {
    const double w = (double)(ntiles * s) / NCU;
    if (w / std::ceil(w) >= 0.8) return s;
  }
  return 8;
}

size_t smem_bytes() { return (size_t)4 * HT * HROW * sizeof(uint16_t); }

}  // namespace

size_t hessian_workspace_bytes(int64_t n, int64_t d) {
  const int64_t T = (d + HT - 1) / HT, ntiles = T * (T + 1) / 2;
  const int S = choose_splits(ntiles, n);
  if (S <= 1) return 0;
  return (size_t)ntiles * S * HT * HT * sizeof(float) + (size_t)ntiles * sizeof(int) + 256;
}

hipError_t hessian_f16(float* H, int64_t d, const void* X, int dtype, int64_t n, int64_t ldx, void* work,
                       size_t work_bytes, hipStream_t s) {
  if (n <= 0 || d <= 0) return hipSuccess;
  HessArgs a{};
  a.H = H;
  a.d = d;
  a.X = static_cast<const uint16_t*>(X);
  a.n = n;
  a.ldx = ldx;
  a.T = (int)((d + HT - 1) / HT);
  const int64_t ntiles = (int64_t)a.T * (a.T + 1) / 2;
  a.ntiles = (int)ntiles;
  int S = choose_splits(ntiles, n);
  const size_t need = hessian_workspace_bytes(n, d);
  if (S > 1 && (work == nullptr || work_bytes < need)) S = 1;  // correct, fewer workgroups
  a.S = S;
  a.per_xcd = (int)((ntiles + 7) / 8);
  const int64_t grid = S > 1 ? ntiles * S : 8 * (int64_t)a.per_xcd;
  a.split_len = ((n + S - 1) / S + HK - 1) / HK * HK;
  a.vec = ((uintptr_t)X % 16 == 0) && (ldx % 8 == 0);
  if (S > 1) {
    a.partial = static_cast<float*>(work);
    a.counters = reinterpret_cast<int*>(static_cast<char*>(work) + (size_t)ntiles * S * HT * HT * sizeof(float));
    hipLaunchKernelGGL(zero_ints, dim3((unsigned)((ntiles + 255) / 256)), dim3(256), 0, s, a.counters, (int)ntiles);
  }
  const size_t sm = smem_bytes();
  if (dtype == F16) {
    static bool attr_f16 = false;
    if (!attr_f16) {
      (void)hipFuncSetAttribute((const void*)hess_kernel<half8>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm);
      attr_f16 = true;
    }
    hipLaunchKernelGGL(hess_kernel<half8>, dim3((unsigned)grid), dim3(256), sm, s, a);
  } else {
    static bool attr_bf16 = false;
    if (!attr_bf16) {
      (void)hipFuncSetAttribute((const void*)hess_kernel<bf16x8>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm);
      attr_bf16 = true;
    }
    hipLaunchKernelGGL(hess_kernel<bf16x8>, dim3((unsigned)grid), dim3(256), sm, s, a);
  }
  return hipGetLastError();
}

}  // namespace gptq
