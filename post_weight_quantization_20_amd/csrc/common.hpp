// Shared device helpers and the internal launcher interface of the GPTQ layer-solver library.
// CDNA4 (gfx950) only: wave64, MFMA matrix cores, 160 KB LDS per CU.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>
#include <stdint.h>
#include <stddef.h>

#include "../../include/gptq.h"

#define GPTQ_DEV __device__ __forceinline__

namespace gptq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

enum DType { F32 = 0, F16 = 1, BF16 = 2 };

// ------------------------------------------------------------------ element conversion
GPTQ_DEV float bf16_bits_to_f32(uint16_t b) { return __builtin_bit_cast(float, (uint32_t)b << 16); }

GPTQ_DEV float load_as_f32(const void* p, int dtype, int64_t idx) {
  if (dtype == F32) return static_cast<const float*>(p)[idx];
  if (dtype == F16) return (float)static_cast<const _Float16*>(p)[idx];
  return bf16_bits_to_f32(static_cast<const uint16_t*>(p)[idx]);
}

// ------------------------------------------------------------------ the quantization grid
// Min/max grid of one group. Asymmetric: scale = max(wmax - wmin, 1e-8) / maxq,
// zero = round(-wmin / scale) (GPTQ tools page, "A minimal Python sketch"; round half to even).
// Symmetric (tools page, "Optional refinements"; the Technical Guide's signed int4 range [-8, 7]):
// the same recipe on [-m, m] with m = max(|wmin|, |wmax|), scale = max(2 m, 1e-8) / maxq, and the
// zero fixed at the middle code (maxq + 1) / 2. rs is the correctly rounded reciprocal of the
// scale, used by div_rn.
// The scale as stored in 16 bits (tools page, "Memory arithmetic"): rounded to the nearest float16,
// ties to even, kept positive and finite (the smallest subnormal below, the largest float16 above).
GPTQ_DEV float fp16_scale(float s) {
  const float h = (float)(_Float16)s;
  return fminf(h == 0.0f ? 0x1p-24f : h, 65504.0f);
}

// compact: the grid is what a 16-bit scale and a zero of the code width store, and the loop uses
// exactly that (the scale rounded by fp16_scale, the zero clamped to [0, maxq]).
GPTQ_DEV void make_grid(float wmin, float wmax, float maxq, bool sym, bool compact, float& s, float& z, float& rs) {
  if (sym) {
    const float m = fmaxf(fabsf(wmin), fabsf(wmax));
    s = fmaxf(2.0f * m, 1e-8f) / maxq;
    if (compact) s = fp16_scale(s);
    z = 0.5f * (maxq + 1.0f);
  } else {
    s = fmaxf(wmax - wmin, 1e-8f) / maxq;
    if (compact) s = fp16_scale(s);
    z = rintf(-wmin / s);
    if (compact) z = fminf(fmaxf(z, 0.0f), maxq);
  }
  rs = 1.0f / s;
}

// Correctly rounded w / s from rs = RN(1 / s): one product and one fma-based correction
// (Markstein's division theorem for round-to-nearest with an fma). Equal to the IEEE quotient
// away from overflow and underflow, which the grid's scales (>= 1e-8 / 255) and weights avoid.
GPTQ_DEV float div_rn(float w, float s, float rs) {
  float q0 = w * rs;
  float r = __builtin_fmaf(-q0, s, w);
  return __builtin_fmaf(r, rs, q0);
}

// ------------------------------------------------------------------ lane broadcast
// Calls f(std::integral_constant<int, K>) for K = B .. E-1 (compile-time column indices).
template <int B, int E, typename F>
GPTQ_DEV void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

template <int SRC>
GPTQ_DEV float row_bcast(float v) {
  // DPP row_newbcast: lane SRC of each 16-lane row to the whole row (every lane has a valid
  // source, so no old value is needed)
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x150 + SRC, 0xF, 0xF, true));
}

// DPP row_ror:N - lane i of each 16-lane row takes the value of lane (i + N) mod 16
template <int N>
GPTQ_DEV float row_ror(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x120 + N, 0xF, 0xF, true));
}

// DPP row_ror:15 - lane i of each 16-lane row takes the value of lane (i + 1) mod 16
GPTQ_DEV float row_ror15(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x12F, 0xF, 0xF, false));
}

// ------------------------------------------------------------------ internal launchers

// C[M x N] = alpha * op(A) * op(B) + beta * C, row-major fp32, on MFMA.
// op(A) is A (M x K, lda) or A^T (A stored K x M); op(B) is B (K x N, ldb) or B^T (B stored N x K).
// tri: 0 every element, 1 only elements with m >= n, 2 only m <= n.
// lowerA: op(A) is lower triangular (zero for k > m), so a row tile stops its k loop at its last row.
// batch > 1: `batch` products, the b-th on A + b sA, B + b sB, C + b sC (0 and 1 mean one product).
// beta == 0 never reads C. C must not overlap A or B: several workgroups can share one output
// strip, and one may store while another still reads its operand.
struct GemmArgs {
  int64_t M, N, K;
  const float* A; int64_t lda; int transA;
  const float* B; int64_t ldb; int transB;
  float* C; int64_t ldc;
  float alpha, beta;
  int tri;
  int lowerA;
  int64_t batch, sA, sB, sC;
};
hipError_t gemm_f32(const GemmArgs& a, hipStream_t s);

// H (upper tiles) += 2 X^T X for X = [n x d] fp16 / bf16 (leading dimension ldx) on MFMA.
size_t hessian_workspace_bytes(int64_t n, int64_t d);
hipError_t hessian_f16(float* H, int64_t d, const void* X, int dtype, int64_t n, int64_t ldx,
                       void* work, size_t work_bytes, hipStream_t s, bool overwrite = false);
// H[0:n) = 0 by a fill kernel (no memset, so that the call may be captured in a graph)
hipError_t zero_matrix(float* H, int64_t n, hipStream_t s);

// Factor: damping, processing order and U (see factor.hip). status_dev / info_dev receive device
// addresses of the mean-diagonal check and the first failed pivot (1-based, reversed order).
// one_stream: everything runs on s (no helper stream, event or mutex is created or used).
size_t factor_workspace_bytes(int64_t d);
hipError_t factor(const float* H, int64_t d, int64_t n, double damp, int act_order, float* U, int32_t* perm,
                  void* work, hipStream_t s, int** status_dev, int64_t** info_dev, bool one_stream = false);

// The library's allocation-free scratch (noalloc.hip): the device address of this device's copy of
// a static device array of kNoallocScratchBytes, looked up once per device.
constexpr int64_t kNoallocMaxD = 12288;
constexpr size_t kNoallocScratchBytes =
    256 + ((size_t)kNoallocMaxD * 4 + 255) / 256 * 256 + 4 * (size_t)kNoallocMaxD * 128 * 4;
hipError_t noalloc_scratch(void** ptr);

// Helper streams and events of the current device for work that overlaps within one call (created
// on first use, kept until the process ends; default priority). Hold `mu` while queueing work that
// records or waits on these events: concurrent callers share them.
struct Helpers {
  hipStream_t stream[2];
  hipEvent_t event[8];
  void* mu;   // std::mutex
};
hipError_t helpers(Helpers** out);
void helpers_lock(Helpers* h);
void helpers_unlock(Helpers* h);

// Column loop workspace layout (see quant.hip).
struct QuantLayout {
  int64_t ldw, bp, ld_err;
  size_t off_wp, off_codes, off_err, off_loss, off_iperm, off_colgrp, total;
};
QuantLayout quant_layout(int64_t rows, int64_t d, int block);
// sym: symmetric grids; static_groups: grids of original column groups fixed before the loop;
// compact: 16-bit scales and zeros clamped to the code width, used as stored.
// part_ms (optional, host double[3]): device time of the call's parts, from events recorded between
// its launches (measurement only; the call then waits for the stream): the column-loop kernels, the
// lazy products across super-blocks, and the rest (working copy, indices, un-permute, loss).
hipError_t quantize(const void* W, int w_dtype, int64_t rows, int64_t d, int64_t ld_w, const float* U,
                    const int32_t* perm, int bits, int64_t g, int B, int sym, int static_groups, int compact,
                    uint8_t* codes, float* scales, int32_t* zeros, int32_t* g_idx, double* loss, void* work,
                    hipStream_t s, double* part_ms = nullptr);
// Field layout (nibbles up to 4 bits, bytes above) and the dense bit stream.
hipError_t pack(const uint8_t* codes, int64_t rows, int64_t d, int bits, int32_t* packed, hipStream_t s);
hipError_t pack_dense(const uint8_t* codes, int64_t rows, int64_t d, int bits, int32_t* packed, hipStream_t s);
// Field layout of the codes taken in a column order; a column gather of a row-major matrix.
hipError_t pack_ordered(const uint8_t* codes, int64_t rows, int64_t d, const int32_t* order, int bits, int32_t* packed,
                        hipStream_t s);
hipError_t permute_columns(const void* in, int64_t m, int64_t d, int64_t ld_in, const int32_t* order, int esz,
                           void* out, int64_t ld_out, hipStream_t s);

// y = x W^T from the packed codes (fields or dense stream), scales, zeros and column groups (see
// dequant.hip). g is the group width (>= 1); gidx may be null (column k in group k / g).
hipError_t dequant_gemm(const void* x, int dtype, int64_t m, int64_t ldx, const int32_t* packed, int bits, int dense,
                        const float* scales, const int32_t* zeros, const int32_t* gidx, int64_t rows, int64_t d,
                        int64_t g, float* y, int64_t ldy, hipStream_t s);

// ------------------------------------------------------------------ fp16 products (gemm_f16.hip)
// C[M x N] = alpha A B^T + beta C with A [M x K], B [N x K] fp16 row-major (k contiguous); K a
// multiple of 64, lda and ldb multiples of 8, A and B 16-byte aligned. beta == 0 never reads C.
// batch > 1: `batch` products, the b-th on A + b sA, B + b sB, C + b sC (sA, sB multiples of 8).
// lower: tiles lying wholly above the diagonal (every n > m) are skipped and their C left as is.
struct GemmF16 {
  int64_t M, N, K;
  const _Float16* A; int64_t lda;
  const _Float16* B; int64_t ldb;
  float* C; int64_t ldc;
  float alpha, beta;
  int64_t batch, sA, sB, sC;
  int lower;
};
hipError_t gemm_f16nt(const GemmF16& a, hipStream_t s);
// Rows of scale * X [n x d] (pitch ldx) as fp16 [hi | hi | lo | 0] (act = 1) or [hi | lo | hi | 0]
// (act = 0), pitch split3_pitch(d) = 3 d rounded up to 64: the operands of an fp32 product A W^T
// formed as one fp16 GEMM. The [hi | lo] half of an act row (from column d) is also the input of a
// split Hessian.
int64_t split3_pitch(int64_t d);
hipError_t split3(const float* X, int64_t n, int64_t d, int64_t ldx, float scale, int act, _Float16* S,
                  hipStream_t s);
// out[0] = max |x| over n floats; part holds kAbsmaxParts floats of scratch.
constexpr int kAbsmaxParts = 1024;
hipError_t absmax(const float* x, int64_t n, float* part, float* out, hipStream_t s);

// ------------------------------------------------------------------ decoder block (block.hip)
// W[r, k] = scales[r, G] (codes[r, k] - zeros[r, G]), G = gidx[k] (or k / g when gidx is null),
// as dense fp32 rows of leading dimension ldw.
hipError_t dequantize(const uint8_t* codes, int64_t rows, int64_t d, const float* scales, const int32_t* zeros,
                      const int32_t* gidx, int64_t g, float* W, int64_t ldw, hipStream_t s);
// Row-wise x / sqrt(mean(x^2) + eps).
hipError_t rmsnorm(const float* x, int64_t m, int64_t d, int64_t ldx, float eps, float* y, int64_t ldy, hipStream_t s);
// Multi-head causal attention over seqs sequences of L tokens; Q, K, V, O are [seqs L x heads dh]
// (leading dimensions ld, ld, ld, ldo; Q and K contiguous, ld = heads dh); S is heads x L x L fp32
// scratch and qk3 holds 2 seqs L heads split3_pitch(dh) halves of scratch.
hipError_t causal_attention(const float* Q, const float* K, const float* V, int64_t seqs, int64_t L, int64_t heads,
                            int64_t dh, int64_t ld, float* O, int64_t ldo, float* S, _Float16* qk3, hipStream_t s);
// y = silu(g) * u elementwise; y may be g.
hipError_t silu_mul(const float* g, const float* u, int64_t n, float* y, hipStream_t s);
hipError_t to_f32(const void* x, int dtype, int64_t n, float* y, hipStream_t s);

// Workspace of gptq_quantize_block: byte offsets of the fp32 activations, one dense weight, the
// stage Hessian (with the fp16 halves of its input and their 2d-wide Hessian) and factor, and the
// Hessian, factor and column-loop workspaces.
struct BlockLayout {
  size_t off_xf, off_xa, off_q, off_k, off_v, off_at, off_h1, off_xm, off_g, off_u, off_s, off_wf, off_h, off_uf,
      off_qk3, off_xs, off_w3, off_mx, off_h2, off_hw, off_fw, off_qw, hess_bytes, factor_bytes, quant_bytes, total;
};
BlockLayout block_layout(const gptq_block_shape_t& sh, const gptq_params_t& p);
int quantize_block(const gptq_block_shape_t& sh, const void* X, int x_dtype, const gptq_params_t& p,
                   int true_sequential, const gptq_block_layer_t* layers, float* Y, float* const* hess, char* work,
                   int64_t* info, hipStream_t s);

}  // namespace gptq
