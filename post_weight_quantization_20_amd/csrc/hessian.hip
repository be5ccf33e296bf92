// Hessian accumulation H += 2 X^T X for fp16 / bf16 activations on CDNA4 matrix cores.
//
// The layer Hessian is proportional to the product of the calibration inputs with their transpose
// and is shared by every row of W (GPTQ tools page, "How it works", Step 3; the sketch forms
// 2 X^T X / n, and the normalisation by n happens when the Hessian is damped).
//
// A 256-thread workgroup (4 wave64s, 2x2) owns a 256x256 tile of H in the upper triangle; each wave
// owns 128x128 (4x4 blocks of v_mfma_f32_32x32x16_{f16,bf16}, 256 accumulators per lane). Products
// of fp16/bf16 values are exact in fp32; accumulation is fp32.
//
// X arrives token-major ([tokens x d], features contiguous) and the product contracts over tokens,
// so each MFMA lane needs 8 consecutive tokens of one feature. The main path streams X straight
// into LDS (buffer_load ... lds, 16 bytes a lane, no registers in between) through a ring of four
// 32-token stages, keeping three stages in flight while the fourth is multiplied, and gives each
// lane its tokens with the transposing LDS read ds_read_b64_tr_b16 (two reads of four tokens).
// Rows of a stage are XOR-swizzled in 16-byte units so that the four token rows one transposing
// read touches fall in distinct banks. Out-of-range tokens and features read as zero through the
// buffer descriptor's range check. A register-staged path (8x8 transposes in registers, then LDS)
// covers X that is not 16-byte aligned or whose width is not a multiple of 8.
//
// When the upper-triangle tiles alone cannot fill the 256 CUs, the token range is split 8 ways.
// Each split writes its partial tile to the workspace and a second kernel adds the partials of
// every tile to H in token order across the whole GPU, so the result does not depend on
// scheduling.
#include "common.hpp"

#include <cmath>

namespace gptq {
namespace {

constexpr int HT = 256;            // tile edge (features)
constexpr int NCU = 256;
constexpr int SPLIT_ALIGN = 64;    // split lengths are multiples of both paths' stage lengths

// register-staged path
constexpr int HK = 64;             // tokens per LDS stage
constexpr int HROW = HK + 8;       // LDS row length in halves (16-byte pad)

// LDS-DMA path
constexpr int DK = 32;             // tokens per stage
constexpr int NST = 4;             // stages in the LDS ring (128 KB; a deeper ring crowds L2)
constexpr int ROWB = HT * 2;       // bytes of one token row of a 256-feature strip
constexpr int STRIPB = DK * ROWB;  // one operand of one stage (16 KB)
constexpr int STAGEB = 2 * STRIPB;

typedef short v4s __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
#define GPTQ_LDS __attribute__((address_space(3)))

struct HessArgs {
  float* H;
  int64_t d;
  const uint16_t* X;   // fp16 or bf16 bit patterns
  int64_t n, ldx;
  int T;               // tiles per dimension
  int ntiles;          // T (T + 1) / 2
  int S;               // token splits: 1 or 8
  int per_xcd;         // S == 1: tiles per XCD (contiguous in the tile order)
  int full;            // S == 8: workgroup slots per XCD that take a whole (tile, split) item,
                       // 32 times the number of whole 32-tile groups
  int q;               // S == 8: parts each remaining item is cut into
  int64_t split_len;   // tokens per split (multiple of SPLIT_ALIGN)
  float* partial;      // S == 8: one HT x HT partial tile per workgroup
  int vec;             // 16-byte loads allowed
  int overwrite;       // H's tiles are set to 2 X^T X instead of added to
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

// Workgroup b runs on XCD b % 8 (32 CUs each). Without token splits, XCD x takes a contiguous run
// of tiles over all tokens. With 8 splits there are 8 ntiles (tile, split) items, ntiles per XCD:
//  - Whole groups first. The tile order is cut into groups of 32 consecutive tiles, and XCD round r
//    of XCD x (its slots 32 r .. 32 r + 31, which run together) takes group j % G of split j / G
//    with j = 8 r + x and G groups in all. A round's 32 workgroups read the same tokens of one split
//    and share its feature strips in the XCD's L2, and the XCDs running the same split at the same
//    time (8 / G of them, or all 8 for G >= 8) read the same token range, so a line one XCD brings
//    in from HBM serves the others' L2 misses from the Infinity Cache.
//  - Then the tiles past the last whole group: XCD x takes them in split x, each cut into q token
//    ranges so that this last, partial round fills the XCD too.
struct Work {
  int tile, split, part, nparts;
  int64_t fa, fb, t_begin, t_end;
  bool diag;
};

GPTQ_DEV bool map_block(const HessArgs& a, Work& w) {
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  int64_t lo, hi;
  if (a.S > 1) {
    if (slot < a.full) {
      const int j = 8 * (slot / 32) + xcd, ngroups = a.full / 32;
      w.split = j / ngroups;
      w.tile = (j % ngroups) * 32 + slot % 32;
      w.part = 0;
      w.nparts = 1;
    } else {
      w.tile = a.full + (slot - a.full) / a.q;
      w.split = xcd;
      w.part = (slot - a.full) % a.q;
      w.nparts = a.q;
      if (w.tile >= a.ntiles) return false;
    }
    lo = (int64_t)w.split * a.split_len;
    hi = lo + a.split_len;
    if (w.nparts > 1) {
      const int64_t plen = (a.split_len / w.nparts + SPLIT_ALIGN - 1) / SPLIT_ALIGN * SPLIT_ALIGN;
      const int64_t end = hi;
      lo = min(end, lo + w.part * plen);
      hi = min(end, lo + plen);
    }
  } else {
    w.tile = xcd * a.per_xcd + slot;
    w.split = w.part = 0;
    w.nparts = 1;
    if (slot >= a.per_xcd || w.tile >= a.ntiles) return false;
    lo = 0;
    hi = a.n;
  }
  int ti, tj;
  tile_at(w.tile, a.T, ti, tj);
  w.diag = ti == tj;
  w.fa = (int64_t)ti * HT;
  w.fb = (int64_t)tj * HT;
  w.t_begin = min(lo, a.n);
  w.t_end = min(hi, a.n);
  return true;
}

// Workgroups holding partials of `tile`, in token order (split, then part).
template <typename F>
GPTQ_DEV void for_each_partial(const HessArgs& a, int tile, F&& f) {
  for (int split = 0; split < a.S; ++split) {
    if (tile < a.full) {
      const int j = split * (a.full / 32) + tile / 32;
      f(8 * (32 * (j / 8) + tile % 32) + j % 8);
    } else {
      for (int p = 0; p < a.q; ++p) f(8 * (a.full + (tile - a.full) * a.q + p) + split);
    }
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

GPTQ_DEV void zero_acc(floatx16 (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
}

// Adds 2 * acc to H (sets H to it with overwrite) when there is one split, or stores the split's
// partial tile for reduce_partials.
// Accumulator register r of lane l holds row 8*(r/4) + 4*(l/32) + r%4, column l%32 of its 32x32
// block.
GPTQ_DEV void finish_tile(const HessArgs& a, const Work& w, const floatx16 (&acc)[4][4]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int li = lane & 31, lk = lane >> 5;
  if (a.S == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t m = w.fa + wm * 128 + i * 32 + 8 * (r >> 2) + 4 * lk + (r & 3);
          const int64_t c = w.fb + wn * 128 + j * 32 + li;
          if (m < a.d && c < a.d) {
            float* h = a.H + m * a.d + c;
            *h = a.overwrite ? 2.0f * acc[i][j][r] : __builtin_fmaf(2.0f, acc[i][j][r], *h);
          }
        }
    return;
  }
  float* part = a.partial + (int64_t)blockIdx.x * (HT * HT);
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
}

// H (upper tiles) += 2 * the sum of each tile's partials in token order (= with overwrite, and H is
// not read). Workgroup (tile, chunk) takes 1024 consecutive elements of one tile, four per thread.
__global__ __launch_bounds__(256) void reduce_partials(HessArgs a) {
  constexpr int CHUNKS = HT * HT / 1024;
  const int tile = blockIdx.x / CHUNKS;
  const int e = (blockIdx.x % CHUNKS) * 1024 + threadIdx.x * 4;
  floatx4 s = {0.0f, 0.0f, 0.0f, 0.0f};
  for_each_partial(a, tile, [&](int b) { s += *reinterpret_cast<const floatx4*>(a.partial + (int64_t)b * HT * HT + e); });
  int ti, tj;
  tile_at(tile, a.T, ti, tj);
  const int64_t gm = (int64_t)ti * HT + e / HT;
  if (gm >= a.d) return;
  const int64_t gc0 = (int64_t)tj * HT + e % HT;
  float* h = a.H + gm * a.d + gc0;
  if (a.d % 4 == 0 && (uintptr_t)a.H % 16 == 0 && gc0 + 4 <= a.d) {   // one 16-byte read-modify-write
    floatx4 v = a.overwrite ? floatx4{0.0f, 0.0f, 0.0f, 0.0f} : *reinterpret_cast<const floatx4*>(h);
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = __builtin_fmaf(2.0f, s[k], v[k]);
    *reinterpret_cast<floatx4*>(h) = v;
    return;
  }
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (gc0 + k < a.d) h[k] = __builtin_fmaf(2.0f, s[k], a.overwrite ? 0.0f : h[k]);
}

// ------------------------------------------------------------------ register-staged path

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
__global__ __launch_bounds__(256) void hess_reg_kernel(HessArgs a) {
  extern __shared__ __align__(16) uint16_t smem[];
  constexpr int TILE = HT * HROW;   // halves per operand tile; buffer [stage][operand]
  Work w;
  if (!map_block(a, w)) return;
  const bool diag = w.diag;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int li = lane & 31, lk = lane >> 5;

  // loader: each thread moves one 8-token x 8-feature block of each operand per stage; 8
  // consecutive lanes take 8 token blocks of one feature block (128-byte global segments,
  // conflict-free 16-byte LDS row stores)
  const int fl = (tid >> 3) * 8, tl = (tid & 7) * 8;

  floatx16 acc[4][4];
  zero_acc(acc);

  u32x4 ra[8], rb[8];
  int64_t t0 = w.t_begin;
  int buf = 0;
  if (t0 < w.t_end) {
    load_block(a, t0 + tl, w.t_end, w.fa + fl, ra);
    if (!diag) load_block(a, t0 + tl, w.t_end, w.fb + fl, rb);
    store_block(smem, fl, tl, ra);
    if (!diag) store_block(smem + TILE, fl, tl, rb);
  }
  __syncthreads();
  for (; t0 < w.t_end; t0 += HK) {
    const bool more = t0 + HK < w.t_end;
    if (more) {
      load_block(a, t0 + HK + tl, w.t_end, w.fa + fl, ra);
      if (!diag) load_block(a, t0 + HK + tl, w.t_end, w.fb + fl, rb);
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
  finish_tile(a, w, acc);
}

// ------------------------------------------------------------------ LDS-DMA path

// Swizzle of the 16-byte units of token row t (XOR on unit-index bits 1..3). The transposing read
// takes 4 consecutive token rows at once (t % 4 = 0..3); their units land in distinct 16-byte bank
// groups for both 16- and 32-lane read phases.
GPTQ_DEV int row_swizzle(int t) {
  t &= 3;
  return (t << 1) ^ (t << 2);
}

// One 16-byte buffer load per lane into LDS: lane j's bytes land at lds_addr + 16 j (lds_addr is
// wave-uniform, in M0; the s_nop is the wait state an M0 write needs before an LDS-DMA load). The
// load is completed by the s_waitcnt vmcnt in stage_barrier; it is written as asm so the compiler
// does not wait for it before every LDS read.
GPTQ_DEV void dma16(i32x4 rsrc, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(lds_addr)
               : "memory");
}

// Waits until at most N of this thread's DMA loads are in flight and all its LDS reads are done,
// then synchronises the workgroup (no memory fence: a fence would drain every load in flight).
template <int N>
GPTQ_DEV void stage_barrier() {
  // the builtin tells the compiler that no LDS read is pending any more (so it adds no waits for
  // them later); the asm waits for the loads, which the compiler does not track
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0), vmcnt and expcnt not waited for
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Barrier once at most `after` stages of this thread's loads (L per stage) are still in flight.
template <int L>
GPTQ_DEV void stage_wait(int after) {
  if (after >= 4) stage_barrier<4 * L>();
  else if (after == 3) stage_barrier<3 * L>();
  else if (after == 2) stage_barrier<2 * L>();
  else if (after == 1) stage_barrier<L>();
  else stage_barrier<0>();
}

template <typename V, bool DIAG>
GPTQ_DEV void dma_tile(const HessArgs& a, const Work& w, floatx16 (&acc)[4][4], GPTQ_LDS char* lds) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int nst = (int)((w.t_end - w.t_begin + DK - 1) / DK);
  const uint32_t lds_base = (uint32_t)(uintptr_t)lds;

  // loader: load q (0..3) of wave v fills token rows 8v + 2q and 8v + 2q + 1 of a stage's strip;
  // lane j takes row (j / 32), 16-byte unit j % 32 in LDS, holding features 8 * (unit ^ swizzle)
  constexpr uint32_t OOB = 0x80000000u;   // beyond any descriptor range: reads as zero
  uint32_t voa[4], vob[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int t = 8 * wave + 2 * q + (lane >> 5);
    const int u = (lane & 31) ^ row_swizzle(t);
    const int64_t f1 = w.fa + 8 * u, f2 = w.fb + 8 * u;
    voa[q] = f1 < a.d ? (uint32_t)((t * a.ldx + f1) * 2) : OOB;
    vob[q] = f2 < a.d ? (uint32_t)((t * a.ldx + f2) * 2) : OOB;
  }
  auto stage_rsrc = [&](int s) {
    const int64_t t = w.t_begin + (int64_t)s * DK;
    const int64_t rows = min((int64_t)DK, w.t_end - t);
    const uint64_t base = (uint64_t)(uintptr_t)(a.X + t * a.ldx);
    const int nrec = (int)(((rows - 1) * a.ldx + a.d) * 2);   // bytes of the stage's valid tokens
    return i32x4{(int)(uint32_t)base, (int)(uint32_t)(base >> 32), nrec, 0x00020000};
  };
  auto stage_dst = [&](int s) { return lds_base + (uint32_t)((s % NST) * STAGEB + wave * 4096); };
  auto issue_a = [&](int s, const i32x4& rs) {
#pragma unroll
    for (int q = 0; q < 4; ++q) dma16(rs, voa[q], stage_dst(s) + q * 1024);
  };
  auto issue_b = [&](int s, const i32x4& rs) {
    if (!DIAG) {
#pragma unroll
      for (int q = 0; q < 4; ++q) dma16(rs, vob[q], stage_dst(s) + STRIPB + q * 1024);
    }
  };
  auto issue = [&](int s) {
    const i32x4 rs = stage_rsrc(s);
    issue_a(s, rs);
    issue_b(s, rs);
  };

  // reader: the transposing read gives lane i of each 16-lane group element i % 4 of the 4-element
  // reads of lanes i / 4 + 4k (k = 0..3). Lane l of the MFMA needs feature l % 32 at tokens
  // 8 (l / 32) .. + 7, so reading lane s takes token row 8 (l / 32) + s / 4 (+4 for the second
  // read), features 16 ((l / 16) % 2) + 4 (s % 4) .. + 3 of its 32-feature block.
  const int g = lane >> 4;
  const int row_lane = ((lane & 15) >> 2) + 8 * (g >> 1);
  const int sw = row_swizzle((lane & 15) >> 2);
  int offa[4], offb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int unit = 4 * i + 2 * (g & 1) + ((lane & 3) >> 1);
    offa[i] = row_lane * ROWB + ((unit ^ sw) + 16 * wm) * 16 + 8 * (lane & 1);
    offb[i] = row_lane * ROWB + ((unit ^ sw) + 16 * wn) * 16 + 8 * (lane & 1) + (DIAG ? 0 : STRIPB);
  }

  // operands of one 16-token step: two transposing reads per 32-feature block (blocks i0..i1-1)
  auto read_step = [&](int stage, int ks, V (&av)[4], V (&bv)[4], int i0 = 0, int i1 = 4) {
    GPTQ_LDS char* buf = lds + (stage % NST) * STAGEB + 16 * ks * ROWB;
#pragma unroll
    for (int i = i0; i < i1; ++i) {
      const v4s a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((GPTQ_LDS v4s*)(buf + offa[i]));
      const v4s a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((GPTQ_LDS v4s*)(buf + offa[i] + 4 * ROWB));
      av[i] = __builtin_bit_cast(V, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
      const v4s b0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((GPTQ_LDS v4s*)(buf + offb[i]));
      const v4s b1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((GPTQ_LDS v4s*)(buf + offb[i] + 4 * ROWB));
      bv[i] = __builtin_bit_cast(V, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };
  auto mma_step = [&](const V (&av)[4], const V (&bv)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma16<V>(av[i], bv[j], acc[i][j]);
  };

  // Every buffer of the ring is filled up front. In iteration `it` the barrier sits between the
  // two 16-token steps of stage `it`: after it, stage it + 1 is complete in LDS (each thread has
  // waited for its own loads of it) and no wave still reads stage `it` (each has waited for its
  // reads), so the loads of stage it + NST go into that buffer while the second step multiplies
  // and the first operands of stage it + 1 are read.
  constexpr int L = DIAG ? 4 : 8;   // loads per thread per stage
  for (int s = 0; s < NST && s < nst; ++s) issue(s);
  if (nst <= 0) return;
  stage_wait<L>(min(NST - 1, nst - 1));
  if (DIAG && wm == 1 && wn == 0) {
    // On a diagonal tile this wave's 128 x 128 quadrant lies below the diagonal, where H is not
    // authoritative: it only loads its share of each stage and meets the barriers, and its sums
    // stay zero (fewer matrix-core cycles for a kernel that the power limit holds back).
    for (int it = 0; it < nst; ++it) {
      stage_wait<L>(min(NST - 2, nst - 2 - it));
      if (it + NST < nst) issue(it + NST);
    }
    return;
  }
  V a0[4], b0[4], a1[4], b1[4];
  read_step(0, 0, a0, b0);
  for (int it = 0; it < nst; ++it) {
    // The first step's operands were read a whole step ago: waiting for them here (instead of
    // after the next reads are queued, where the 15-deep LDS counter would force waiting for those
    // too) lets the reads of the second step run under the first step's MFMAs.
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    read_step(it, 1, a1, b1);
    mma_step(a0, b0);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
    }
    // stages issued after stage it + 1 so far: min(it + NST - 1, nst - 1) - (it + 1)
    stage_wait<L>(min(NST - 2, nst - 2 - it));
    // second step, with the first operands of stage it + 1 read under its MFMAs and the loads of
    // stage it + NST issued half way through (after the last stage those reads take a stale buffer
    // of the ring and are not used)
    const bool more = it + NST < nst;
    read_step(it + 1, 0, a0, b0, 0, 2);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma16<V>(a1[i], b1[j], acc[i][j]);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
    }
    if (more) issue(it + NST);
    read_step(it + 1, 0, a0, b0, 2, 4);
#pragma unroll
    for (int i = 2; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma16<V>(a1[i], b1[j], acc[i][j]);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 2);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 2);
    }
  }
}

template <typename V>
__global__ __launch_bounds__(256) void hess_kernel(HessArgs a) {
  extern __shared__ __align__(16) char smem_raw[];
  Work w;
  if (!map_block(a, w)) return;
  floatx16 acc[4][4];
  zero_acc(acc);
  GPTQ_LDS char* lds = (GPTQ_LDS char*)smem_raw;
  if (w.diag) dma_tile<V, true>(a, w, acc, lds);
  else dma_tile<V, false>(a, w, acc, lds);
  finish_tile(a, w, acc);
}

// Token splits: none when the tiles alone give every CU three or more workgroups or when there are
// too few tokens; otherwise 8 (the partial last round is cut finer, see map_block).
int choose_splits(int64_t ntiles, int64_t n) {
  if (ntiles >= 3 * NCU) return 1;
  if (n < 8 * 16 * HK) return 1;
  return 8;
}

template <typename V>
hipError_t launch(const HessArgs& a, int64_t grid, bool dma, hipStream_t s) {
  static bool attr_set[2] = {false, false};
  const void* fn = dma ? (const void*)hess_kernel<V> : (const void*)hess_reg_kernel<V>;
  const size_t sm = dma ? (size_t)NST * STAGEB : (size_t)4 * HT * HROW * sizeof(uint16_t);
  if (!attr_set[dma]) {
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm);
    if (e != hipSuccess) return e;
    attr_set[dma] = true;
  }
  if (dma) hipLaunchKernelGGL(hess_kernel<V>, dim3((unsigned)grid), dim3(256), sm, s, a);
  else hipLaunchKernelGGL(hess_reg_kernel<V>, dim3((unsigned)grid), dim3(256), sm, s, a);
  return hipGetLastError();
}

struct Plan {
  int T, ntiles, S, per_xcd, full, q;
  int64_t grid, split_len;
};

Plan plan(int64_t n, int64_t d) {
  Plan p{};
  p.T = (int)((d + HT - 1) / HT);
  p.ntiles = p.T * (p.T + 1) / 2;
  p.S = choose_splits(p.ntiles, n);
  p.split_len = ((n + p.S - 1) / p.S + SPLIT_ALIGN - 1) / SPLIT_ALIGN * SPLIT_ALIGN;
  p.per_xcd = (p.ntiles + 7) / 8;
  if (p.S > 1) {
    constexpr int PER = NCU / 8;    // CUs per XCD
    p.full = p.ntiles / PER * PER;    // whole 32-tile groups
    const int r = p.ntiles - p.full;
    p.q = r > 0 ? std::max(1, PER / r) : 1;
    // parts shorter than a few stages are not worth their partial tiles
    while (p.q > 1 && p.split_len / p.q < 8 * SPLIT_ALIGN) --p.q;
    p.grid = 8 * (int64_t)(p.full + r * p.q);
  } else {
    p.grid = 8 * (int64_t)p.per_xcd;
  }
  return p;
}

}  // namespace

size_t hessian_workspace_bytes(int64_t n, int64_t d) {
  const Plan p = plan(n, d);
  if (p.S <= 1) return 0;
  return (size_t)p.grid * HT * HT * sizeof(float);
}

namespace {
__global__ __launch_bounds__(256) void zero_f32(float* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0.0f;
}
}  // namespace

hipError_t zero_matrix(float* H, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_f32, dim3((unsigned)std::min<int64_t>((n + 255) / 256, 65536)), dim3(256), 0, s, H, n);
  return hipGetLastError();
}

hipError_t hessian_f16(float* H, int64_t d, const void* X, int dtype, int64_t n, int64_t ldx, void* work,
                       size_t work_bytes, hipStream_t s, bool overwrite) {
  if (n <= 0 || d <= 0) return hipSuccess;
  Plan p = plan(n, d);
  if (p.S > 1 && (work == nullptr || work_bytes < hessian_workspace_bytes(n, d))) {
    // correct with fewer workgroups: no token splits
    p.S = 1;
    p.split_len = n;
    p.grid = 8 * (int64_t)p.per_xcd;
  }
  HessArgs a{};
  a.H = H;
  a.d = d;
  a.X = static_cast<const uint16_t*>(X);
  a.n = n;
  a.ldx = ldx;
  a.T = p.T;
  a.ntiles = p.ntiles;
  a.S = p.S;
  a.per_xcd = p.per_xcd;
  a.full = p.full;
  a.q = p.q;
  a.split_len = p.split_len;
  a.vec = ((uintptr_t)X % 16 == 0) && (ldx % 8 == 0);
  a.overwrite = overwrite ? 1 : 0;
  // the DMA path needs 16-byte units that never straddle the end of a row, and 32-bit offsets
  // within a stage
  const bool dma = a.vec && d % 8 == 0 && (int64_t)DK * ldx * 2 < ((int64_t)1 << 31);
  if (p.S > 1) a.partial = static_cast<float*>(work);
  const hipError_t e = dtype == F16 ? launch<half8>(a, p.grid, dma, s) : launch<bf16x8>(a, p.grid, dma, s);
  if (e != hipSuccess || p.S == 1) return e;
  hipLaunchKernelGGL(reduce_partials, dim3((unsigned)((int64_t)p.ntiles * (HT * HT / 1024))), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace gptq
