// C-ABI entry points: host-side argument checks, then launches on the caller's stream.
#include <cmath>
#include <cstring>

#include "../../include/gptq.h"
#include "common.hpp"


namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 31;  // d * d and rows * d stay far inside int64

bool dtype_ok(int32_t t) { return t == GPTQ_F32 || t == GPTQ_F16 || t == GPTQ_BF16; }

// Validates the settings shared by factor and quantize. Returns GPTQ_OK or the error.
gptq_status_t check_params(const gptq_params_t* p, int64_t d, bool quant) {
  if (!p) return GPTQ_EINVAL;
  if ((p->sym != 0 && p->sym != 1) || (p->static_groups != 0 && p->static_groups != 1) ||
      (p->compact_meta != 0 && p->compact_meta != 1))
    return GPTQ_EINVAL;
  if (p->act_order != 0 && p->act_order != 1) return GPTQ_EINVAL;
  if (!(p->damp >= 0.0) || !std::isfinite(p->damp)) return GPTQ_EINVAL;
  if (!quant) return GPTQ_OK;
  if (p->bits < 2 || p->bits > 8) return GPTQ_EINVAL;
  if (p->block_size < 1) return GPTQ_EINVAL;
  if (p->block_size > 128) return GPTQ_EUNSUPPORTED;
  const int64_t g = p->group_size <= 0 ? d : p->group_size;
  if (g == 1) return GPTQ_EINVAL;
  if (g < d && !(p->block_size % g == 0 || g % p->block_size == 0)) return GPTQ_EINVAL;
  return GPTQ_OK;
}

gptq_status_t hip_status(hipError_t e) { return e == hipSuccess ? GPTQ_OK : GPTQ_EHIP; }

}  // namespace

extern "C" {

const char* gptq_status_string(gptq_status_t s) {
  switch (s) {
    case GPTQ_OK: return "ok";
    case GPTQ_EINVAL: return "invalid argument";
    case GPTQ_ENOTPD: return "damped Hessian is not positive definite";
    case GPTQ_EUNSUPPORTED: return "unsupported setting";
    case GPTQ_EHIP: return "HIP runtime error";
    case GPTQ_ENOMEM: return "workspace too small";
    default: return "unknown status";
  }
}

size_t gptq_workspace_bytes(int32_t kind, int64_t a, int64_t d, const gptq_params_t* p) {
  if (d <= 0 || d > kMaxDim || a < 0 || a > kMaxDim) return 0;
  switch (kind) {
    case GPTQ_WS_HESSIAN: return gptq::hessian_workspace_bytes(a, d);
    case GPTQ_WS_FACTOR: return gptq::factor_workspace_bytes(d);
    case GPTQ_WS_QUANTIZE: {
      if (!p || p->block_size < 1 || p->block_size > 128) return 0;
      return gptq::quant_layout(a, d, p->block_size).total;
    }
    default: return 0;
  }
}

}  // extern "C"

namespace {

// gptq_hessian_accumulate (H += 2 X^T X) and gptq_hessian_compute (H = 2 X^T X)
gptq_status_t hessian_call(float* H, int64_t d, const void* X, int32_t x_dtype, int64_t n_tok, int64_t ld_x,
                           void* work, size_t work_bytes, void* stream, bool overwrite) {
  if (!H || d <= 0 || d > kMaxDim || n_tok < 0 || n_tok > kMaxDim || !dtype_ok(x_dtype)) return GPTQ_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (n_tok == 0) return overwrite ? hip_status(gptq::zero_matrix(H, d * d, s)) : GPTQ_OK;
  if (!X || ld_x < d) return GPTQ_EINVAL;
  if (x_dtype == GPTQ_F32) {
    gptq::GemmArgs a{};
    a.M = d; a.N = d; a.K = n_tok;
    a.A = static_cast<const float*>(X); a.lda = ld_x; a.transA = 1;
    a.B = static_cast<const float*>(X); a.ldb = ld_x; a.transB = 0;
    a.C = H; a.ldc = d;
    a.alpha = 2.0f; a.beta = overwrite ? 0.0f : 1.0f; a.tri = 2;
    return hip_status(gptq::gemm_f32(a, s));
  }
  return hip_status(gptq::hessian_f16(H, d, X, x_dtype, n_tok, ld_x, work, work_bytes, s, overwrite));
}

}  // namespace

extern "C" {

gptq_status_t gptq_hessian_accumulate(float* H, int64_t d, const void* X, int32_t x_dtype, int64_t n_tok,
                                      int64_t ld_x, void* work, size_t work_bytes, void* stream) {
  return hessian_call(H, d, X, x_dtype, n_tok, ld_x, work, work_bytes, stream, false);
}

gptq_status_t gptq_hessian_compute(float* H, int64_t d, const void* X, int32_t x_dtype, int64_t n_tok,
                                   int64_t ld_x, void* work, size_t work_bytes, void* stream) {
  return hessian_call(H, d, X, x_dtype, n_tok, ld_x, work, work_bytes, stream, true);
}

}  // extern "C"

namespace {

// The checks and the call shared by gptq_factor and gptq_factor_noalloc: work is the workspace (the
// caller's, or the static scratch), one_stream keeps every launch on the caller's stream.
gptq_status_t factor_call(const float* H, int64_t d, int64_t n_total, const gptq_params_t* p, float* U,
                          int32_t* perm, void* work, int64_t* info, hipStream_t s, bool one_stream) {
  int* status_dev = nullptr;
  int64_t* info_dev = nullptr;
  hipError_t e = gptq::factor(H, d, n_total, p->damp, p->act_order, U, perm, work, s, &status_dev, &info_dev,
                              one_stream);
  if (e != hipSuccess) return GPTQ_EHIP;
  int64_t dev_info = 0;
  int dev_status = 0;
  if (hipMemcpyAsync(&dev_info, info_dev, sizeof(dev_info), hipMemcpyDeviceToHost, s) != hipSuccess) return GPTQ_EHIP;
  if (hipMemcpyAsync(&dev_status, status_dev, sizeof(dev_status), hipMemcpyDeviceToHost, s) != hipSuccess)
    return GPTQ_EHIP;
  if (hipStreamSynchronize(s) != hipSuccess) return GPTQ_EHIP;
  // the factorization runs on the reversed order; report the processing-order column (1-based)
  *info = dev_info > 0 ? d - dev_info + 1 : 0;
  if (dev_status != 0) return GPTQ_EINVAL;
  return dev_info != 0 ? GPTQ_ENOTPD : GPTQ_OK;
}

gptq_status_t factor_args(const float* H, int64_t d, int64_t n_total, const gptq_params_t* p, const float* U,
                          const int32_t* perm, const int64_t* info) {
  if (!H || !U || !perm || !info || d <= 0 || d > kMaxDim || n_total <= 0) return GPTQ_EINVAL;
  gptq_status_t st = check_params(p, d, false);
  if (st != GPTQ_OK) return st;
  const char* h0 = reinterpret_cast<const char*>(H);
  const char* u0 = reinterpret_cast<const char*>(U);
  const size_t bytes = (size_t)d * d * sizeof(float);
  if (h0 != u0 && h0 < u0 + bytes && u0 < h0 + bytes) return GPTQ_EINVAL;   // in place, or apart
  return GPTQ_OK;
}

}  // namespace

extern "C" {

gptq_status_t gptq_factor(const float* H, int64_t d, int64_t n_total, const gptq_params_t* p, float* U,
                          int32_t* perm, void* work, size_t work_bytes, int64_t* info, void* stream) {
  gptq_status_t st = factor_args(H, d, n_total, p, U, perm, info);
  if (st != GPTQ_OK) return st;
  if (!work) return GPTQ_EINVAL;
  if (work_bytes < gptq::factor_workspace_bytes(d)) return GPTQ_ENOMEM;
  return factor_call(H, d, n_total, p, U, perm, work, info, static_cast<hipStream_t>(stream), false);
}

gptq_status_t gptq_factor_noalloc(const float* H, int64_t d, int64_t n_total, const gptq_params_t* p, float* U,
                                  int32_t* perm, int64_t* info, void* stream) {
  gptq_status_t st = factor_args(H, d, n_total, p, U, perm, info);
  if (st != GPTQ_OK) return st;
  if (d > GPTQ_FACTOR_NOALLOC_MAX_D) return GPTQ_EUNSUPPORTED;
  static_assert(GPTQ_FACTOR_NOALLOC_MAX_D == gptq::kNoallocMaxD, "scratch sized for another maximum");
  if (gptq::factor_workspace_bytes(d) > gptq::kNoallocScratchBytes) return GPTQ_EUNSUPPORTED;
  void* scratch = nullptr;
  if (gptq::noalloc_scratch(&scratch) != hipSuccess) return GPTQ_EHIP;
  return factor_call(H, d, n_total, p, U, perm, scratch, info, static_cast<hipStream_t>(stream), true);
}

}  // extern "C"

namespace {

gptq_status_t quantize_call(const void* W, int32_t w_dtype, int64_t rows, int64_t d, int64_t ld_w, const float* U,
                            const int32_t* perm, const gptq_params_t* p, uint8_t* codes, float* scales,
                            int32_t* zeros, int32_t* g_idx, double* loss, void* work, size_t work_bytes,
                            void* stream, double* part_ms) {
  if (rows < 0 || rows > kMaxDim || d <= 0 || d > kMaxDim || !dtype_ok(w_dtype)) return GPTQ_EINVAL;
  if (!U || !perm || !g_idx || !loss || !work) return GPTQ_EINVAL;
  if (rows > 0 && (!W || !codes || !scales || !zeros || ld_w < d)) return GPTQ_EINVAL;
  gptq_status_t st = check_params(p, d, true);
  if (st != GPTQ_OK) return st;
  if (work_bytes < gptq::quant_layout(rows, d, p->block_size).total) return GPTQ_ENOMEM;
  const int64_t g = p->group_size <= 0 ? d : p->group_size;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(gptq::quantize(W, w_dtype, rows, d, ld_w, U, perm, p->bits, g, p->block_size, p->sym,
                                   p->static_groups, p->compact_meta, codes, scales, zeros, g_idx, loss, work, s,
                                   part_ms));
}

}  // namespace

extern "C" {

gptq_status_t gptq_quantize_layer(const void* W, int32_t w_dtype, int64_t rows, int64_t d, int64_t ld_w,
                                  const float* U, const int32_t* perm, const gptq_params_t* p, uint8_t* codes,
                                  float* scales, int32_t* zeros, int32_t* g_idx, double* loss, void* work,
                                  size_t work_bytes, void* stream) {
  return quantize_call(W, w_dtype, rows, d, ld_w, U, perm, p, codes, scales, zeros, g_idx, loss, work, work_bytes,
                       stream, nullptr);
}

gptq_status_t gptq_quantize_layer_timed(const void* W, int32_t w_dtype, int64_t rows, int64_t d, int64_t ld_w,
                                        const float* U, const int32_t* perm, const gptq_params_t* p, uint8_t* codes,
                                        float* scales, int32_t* zeros, int32_t* g_idx, double* loss, void* work,
                                        size_t work_bytes, double* part_ms, void* stream) {
  if (!part_ms) return GPTQ_EINVAL;
  return quantize_call(W, w_dtype, rows, d, ld_w, U, perm, p, codes, scales, zeros, g_idx, loss, work, work_bytes,
                       stream, part_ms);
}

gptq_status_t gptq_pack(const uint8_t* codes, int64_t rows, int64_t d, int32_t bits, int32_t* packed, void* stream) {
  if (rows < 0 || rows > kMaxDim || d < 8 || d > kMaxDim || d % 8 != 0 || bits < 1 || bits > 8) return GPTQ_EINVAL;
  if (rows == 0) return GPTQ_OK;
  if (!codes || !packed) return GPTQ_EINVAL;
  return hip_status(gptq::pack(codes, rows, d, bits, packed, static_cast<hipStream_t>(stream)));
}

gptq_status_t gptq_pack_dense(const uint8_t* codes, int64_t rows, int64_t d, int32_t bits, int32_t* packed,
                              void* stream) {
  if (rows < 0 || rows > kMaxDim || d < 1 || d > kMaxDim || bits < 1 || bits > 8 || (d * bits) % 32 != 0)
    return GPTQ_EINVAL;
  if (rows == 0) return GPTQ_OK;
  if (!codes || !packed) return GPTQ_EINVAL;
  return hip_status(gptq::pack_dense(codes, rows, d, bits, packed, static_cast<hipStream_t>(stream)));
}

gptq_status_t gptq_pack_ordered(const uint8_t* codes, int64_t rows, int64_t d, int32_t bits, const int32_t* order,
                                int32_t* packed, void* stream) {
  if (rows < 0 || rows > kMaxDim || d < 8 || d > kMaxDim || d % 8 != 0 || bits < 1 || bits > 8) return GPTQ_EINVAL;
  if (rows == 0) return GPTQ_OK;
  if (!codes || !order || !packed) return GPTQ_EINVAL;
  return hip_status(gptq::pack_ordered(codes, rows, d, order, bits, packed, static_cast<hipStream_t>(stream)));
}

gptq_status_t gptq_permute_columns(const void* in, int32_t dtype, int64_t m, int64_t d, int64_t ld_in,
                                   const int32_t* order, void* out, int64_t ld_out, void* stream) {
  if (m < 0 || m > kMaxDim || d < 1 || d > kMaxDim || !dtype_ok(dtype) || ld_in < d || ld_out < d) return GPTQ_EINVAL;
  if (m == 0) return GPTQ_OK;
  if (!in || !order || !out) return GPTQ_EINVAL;
  const int esz = dtype == GPTQ_F32 ? 4 : 2;
  const char* i0 = static_cast<const char*>(in);
  const char* o0 = static_cast<const char*>(out);
  const int64_t in_bytes = ((m - 1) * ld_in + d) * esz, out_bytes = ((m - 1) * ld_out + d) * esz;
  if (i0 < o0 + out_bytes && o0 < i0 + in_bytes) return GPTQ_EINVAL;   // in place would race
  return hip_status(gptq::permute_columns(in, m, d, ld_in, order, esz, out, ld_out, static_cast<hipStream_t>(stream)));
}

gptq_status_t gptq_dequant_gemm(const void* x, int32_t x_dtype, int64_t m, int64_t ld_x, const int32_t* packed,
                                int32_t bits, int32_t layout, const float* scales, const int32_t* zeros,
                                const int32_t* g_idx, int64_t rows, int64_t d, int32_t group_size, float* y,
                                int64_t ld_y, void* stream) {
  if (m < 0 || m > kMaxDim || rows < 0 || rows > kMaxDim || d < 8 || d > kMaxDim || d % 8 != 0) return GPTQ_EINVAL;
  if (!dtype_ok(x_dtype) || ld_x < d || ld_x > kMaxDim || ld_y < rows || ld_y > kMaxDim) return GPTQ_EINVAL;
  if (bits < 1 || bits > 8) return GPTQ_EINVAL;
  if (layout != GPTQ_LAYOUT_FIELDS && layout != GPTQ_LAYOUT_DENSE) return GPTQ_EINVAL;
  if (layout == GPTQ_LAYOUT_DENSE && (d * bits) % 32 != 0) return GPTQ_EINVAL;
  if (m == 0 || rows == 0) return GPTQ_OK;
  if (!x || !packed || !scales || !zeros || !y) return GPTQ_EINVAL;
  const int64_t g = group_size <= 0 ? d : group_size;
  return hip_status(gptq::dequant_gemm(x, x_dtype, m, ld_x, packed, bits, layout == GPTQ_LAYOUT_DENSE, scales, zeros,
                                       g_idx, rows, d, g, y, ld_y, static_cast<hipStream_t>(stream)));
}

namespace {

bool block_shape_ok(const gptq_block_shape_t* sh) {
  if (!sh) return false;
  if (sh->hidden < 8 || sh->hidden > kMaxDim || sh->inter < 8 || sh->inter > kMaxDim) return false;
  if (sh->heads < 1 || sh->heads > 65535 || sh->hidden % sh->heads != 0) return false;
  if (sh->seqs < 1 || sh->seq_len < 1 || sh->seq_len > kMaxDim || sh->seqs > kMaxDim / sh->seq_len) return false;
  if (sh->heads * sh->seq_len > kMaxDim) return false;   // softmax rows of one sequence, one workgroup each
  return std::isfinite(sh->eps) && sh->eps >= 0.0;
}

}  // namespace

size_t gptq_block_workspace_bytes(const gptq_block_shape_t* shape, const gptq_params_t* p) {
  if (!block_shape_ok(shape) || !p || p->block_size < 1 || p->block_size > 128) return 0;
  return gptq::block_layout(*shape, *p).total;
}

gptq_status_t gptq_quantize_block(const gptq_block_shape_t* shape, const void* X, int32_t x_dtype,
                                  const gptq_params_t* p, int32_t true_sequential, const gptq_block_layer_t* layers,
                                  float* Y, float* const* hess, void* work, size_t work_bytes, int64_t* info,
                                  void* stream) {
  if (info) info[0] = -1, info[1] = 0;
  if (!block_shape_ok(shape) || !X || !dtype_ok(x_dtype) || !layers || !Y || !work || !info) return GPTQ_EINVAL;
  if (true_sequential != 0 && true_sequential != 1) return GPTQ_EINVAL;
  gptq_status_t st = check_params(p, std::min(shape->hidden, shape->inter), true);
  if (st != GPTQ_OK) return st;
  if ((st = check_params(p, std::max(shape->hidden, shape->inter), true)) != GPTQ_OK) return st;
  for (int i = 0; i < 7; ++i) {
    const gptq_block_layer_t& l = layers[i];
    if (!l.W || !l.codes || !l.scales || !l.zeros || !l.g_idx || !l.perm || !l.loss || !dtype_ok(l.w_dtype))
      return GPTQ_EINVAL;
  }
  if (work_bytes < gptq::block_layout(*shape, *p).total) return GPTQ_ENOMEM;
  return gptq::quantize_block(*shape, X, x_dtype, *p, true_sequential, layers, Y, hess, static_cast<char*>(work),
                              info, static_cast<hipStream_t>(stream));
}

}  // extern "C"
