// The forward pass a true-sequential block driver needs between quantization steps.
//
// GPTQ tools page, "How it works", Step 9: a block is quantized layer by layer, and with "true
// sequential" ordering the attention projections come first and the inputs of the following layers
// are recomputed through the layers already quantized. The block here is a pre-norm decoder block
// (the pages do not fix one): RMSNorm, multi-head causal self-attention, a residual, RMSNorm, and a
// SiLU-gated MLP. These kernels compute its pieces in fp32:
//   dequantize_kernel      W[r, k] = s[r, G(k)] (q[r, k] - z[r, G(k)]) as dense fp32
//   rmsnorm_kernel         y = x / sqrt(mean(x^2) + eps), one workgroup per row
//   causal_softmax_kernel  row i of S: softmax of scale * S[i, 0..i], zeros after i
//   silu_mul_kernel        y = g / (1 + exp(-g)) * u
//   to_f32_kernel          a fp32 copy of fp32 / fp16 / bf16 values
// Products (x W^T, the attention scores and P V) run on gemm_f32. quantize_block (the body of
// gptq_quantize_block) strings them together with the library's own Hessian, factor and column-loop
// entry points.
#include <hip/hip_runtime.h>

#include <cmath>

#include "../../include/gptq.h"
#include "common.hpp"

namespace gptq {
namespace {

__global__ __launch_bounds__(256) void dequantize_kernel(const uint8_t* __restrict__ codes, int64_t rows, int64_t d,
                                                         const float* __restrict__ scales,
                                                         const int32_t* __restrict__ zeros,
                                                         const int32_t* __restrict__ gidx, int64_t g,
                                                         int64_t ngroups, float* __restrict__ W, int64_t ldw) {
  const int64_t total = rows * d;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int64_t r = e / d, k = e - r * d;
    int64_t G = gidx ? (int64_t)gidx[k] : k / g;
    G = G < 0 ? 0 : G >= ngroups ? ngroups - 1 : G;   // out-of-range entries are clamped
    const int32_t q = codes[e];
    W[r * ldw + k] = scales[r * ngroups + G] * (float)(q - zeros[r * ngroups + G]);
  }
}

// Sum over the workgroup's 256 threads.
GPTQ_DEV float block_sum(float v, float* red) {
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) v += __shfl_xor(v, m, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  const float t = red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  return t;
}

__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ x, int64_t d, int64_t ldx,
                                                      float eps, float* __restrict__ y, int64_t ldy) {
  __shared__ float red[4];
  const float* xr = x + (int64_t)blockIdx.x * ldx;
  float* yr = y + (int64_t)blockIdx.x * ldy;
  float ss = 0.f;
  for (int64_t k = threadIdx.x; k < d; k += 256) ss = __builtin_fmaf(xr[k], xr[k], ss);
  const float inv = 1.0f / sqrtf(block_sum(ss, red) / (float)d + eps);
  for (int64_t k = threadIdx.x; k < d; k += 256) yr[k] = xr[k] * inv;
}

// One row of a stack of L x L score blocks (row r is query i = r mod L of its block, leading
// dimension L): p_j = exp(scale s_j - max) / sum over j <= i, and 0 for j > i (the causal mask).
// Only entries j <= i are read.
__global__ __launch_bounds__(256) void causal_softmax_kernel(float* __restrict__ S, int64_t L, float scale) {
  __shared__ float red[4];
  const int64_t i = (int64_t)blockIdx.x % L;
  float* row = S + (int64_t)blockIdx.x * L;
  float mx = -INFINITY;
  for (int64_t j = threadIdx.x; j <= i; j += 256) mx = fmaxf(mx, scale * row[j]);
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) mx = fmaxf(mx, __shfl_xor(mx, m, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float sum = 0.f;
  for (int64_t j = threadIdx.x; j <= i; j += 256) {
    const float p = expf(scale * row[j] - mx);
    row[j] = p;
    sum += p;
  }
  const float inv = 1.0f / block_sum(sum, red);
  for (int64_t j = threadIdx.x; j < L; j += 256) row[j] = j <= i ? row[j] * inv : 0.0f;
}

// The same softmax with the row held in registers (NPT scores per thread, L <= 256 NPT): the scores
// j <= i are read once and the row is written once.
template <int NPT>
__global__ __launch_bounds__(256) void causal_softmax_reg_kernel(float* __restrict__ S, int64_t L, float scale) {
  __shared__ float red[4];
  const int64_t i = (int64_t)blockIdx.x % L;
  float* row = S + (int64_t)blockIdx.x * L;
  float v[NPT];
  float mx = -INFINITY;
#pragma unroll
  for (int c = 0; c < NPT; ++c) {
    const int64_t j = threadIdx.x + 256 * c;
    v[c] = j <= i ? scale * row[j] : -INFINITY;
    mx = fmaxf(mx, v[c]);
  }
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) mx = fmaxf(mx, __shfl_xor(mx, m, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float sum = 0.f;
#pragma unroll
  for (int c = 0; c < NPT; ++c) {
    const int64_t j = threadIdx.x + 256 * c;
    v[c] = j <= i ? expf(v[c] - mx) : 0.0f;
    sum += v[c];
  }
  const float inv = 1.0f / block_sum(sum, red);
#pragma unroll
  for (int c = 0; c < NPT; ++c) {
    const int64_t j = threadIdx.x + 256 * c;
    if (j < L) row[j] = v[c] * inv;
  }
}

// y may be g itself (each element reads its own g and u before writing)
__global__ __launch_bounds__(256) void silu_mul_kernel(const float* g, const float* __restrict__ u, int64_t n,
                                                       float* y) {
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) {
    const float a = g[e];
    y[e] = a / (1.0f + expf(-a)) * u[e];
  }
}

__global__ __launch_bounds__(256) void to_f32_kernel(const void* __restrict__ x, int dtype, int64_t n,
                                                     float* __restrict__ y) {
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256)
    y[e] = load_as_f32(x, dtype, e);
}

// H = hi^T hi + hi^T lo + lo^T hi + lo^T lo from the upper triangle of the 2d x 2d H2 of [hi | lo]:
// H[i, j] = H2[i, j] + H2[i, d + j] + H2[j, d + i] + H2[d + i, d + j] for i <= j (all four entries lie
// on or above H2's diagonal), in that order; 0 below the diagonal.
__global__ __launch_bounds__(256) void fold_split_kernel(const float* __restrict__ H2, int64_t d,
                                                         float* __restrict__ H) {
  const int64_t total = d * d, l2 = 2 * d;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int64_t i = e / d, j = e - i * d;
    float v = 0.0f;
    if (j >= i) v = ((H2[i * l2 + j] + H2[i * l2 + d + j]) + H2[j * l2 + d + i]) + H2[(d + i) * l2 + d + j];
    H[e] = v;
  }
}

unsigned grid_for(int64_t n) { return (unsigned)std::min<int64_t>((n + 255) / 256, 65536); }

}  // namespace

hipError_t dequantize(const uint8_t* codes, int64_t rows, int64_t d, const float* scales, const int32_t* zeros,
                      const int32_t* gidx, int64_t g, float* W, int64_t ldw, hipStream_t s) {
  if (rows * d <= 0) return hipSuccess;
  hipLaunchKernelGGL(dequantize_kernel, dim3(grid_for(rows * d)), dim3(256), 0, s, codes, rows, d, scales, zeros, gidx,
                     g, (d + g - 1) / g, W, ldw);
  return hipGetLastError();
}

hipError_t rmsnorm(const float* x, int64_t m, int64_t d, int64_t ldx, float eps, float* y, int64_t ldy, hipStream_t s) {
  if (m <= 0) return hipSuccess;
  hipLaunchKernelGGL(rmsnorm_kernel, dim3((unsigned)m), dim3(256), 0, s, x, d, ldx, eps, y, ldy);
  return hipGetLastError();
}

// One sequence at a time, every head in one batched product. The scores S_h = Q_h K_h^T run on the
// split fp16 GEMM: Q and K, viewed as [tokens x heads] rows of dh, are split once per call into
// [hi | hi | lo] and [hi | lo | hi] rows (qk3 holds both), and tiles wholly above the diagonal are
// skipped (the softmax reads only j <= i). Then the causal softmax over all heads' rows, and
// O_h = P_h V_h in fp32 with the k loop of each row tile stopping at its last row (P is zero above
// the diagonal). S holds heads x L x L floats.
hipError_t causal_attention(const float* Q, const float* K, const float* V, int64_t seqs, int64_t L, int64_t heads,
                            int64_t dh, int64_t ld, float* O, int64_t ldo, float* S, _Float16* qk3, hipStream_t s) {
  const float scale = 1.0f / sqrtf((float)dh);
  const int64_t n = seqs * L, kq = split3_pitch(dh);
  _Float16* q3 = qk3;
  _Float16* k3 = qk3 + n * heads * kq;
  hipError_t e = split3(Q, n * heads, dh, dh, 1.0f, 1, q3, s);
  if (e != hipSuccess) return e;
  if ((e = split3(K, n * heads, dh, dh, 1.0f, 0, k3, s)) != hipSuccess) return e;
  for (int64_t sq = 0; sq < seqs; ++sq) {
    const int64_t off = sq * L * ld, off3 = sq * L * heads * kq;
    GemmF16 a{};
    a.M = L; a.N = L; a.K = kq;
    a.A = q3 + off3; a.lda = heads * kq;
    a.B = k3 + off3; a.ldb = heads * kq;
    a.C = S; a.ldc = L;
    a.alpha = 1.0f; a.beta = 0.0f;
    a.batch = heads; a.sA = kq; a.sB = kq; a.sC = L * L;
    a.lower = 1;
    if ((e = gemm_f16nt(a, s)) != hipSuccess) return e;
    const dim3 rows_grid((unsigned)(heads * L));
    if (L <= 512)
      hipLaunchKernelGGL(causal_softmax_reg_kernel<2>, rows_grid, dim3(256), 0, s, S, L, scale);
    else if (L <= 2048)
      hipLaunchKernelGGL(causal_softmax_reg_kernel<8>, rows_grid, dim3(256), 0, s, S, L, scale);
    else
      hipLaunchKernelGGL(causal_softmax_kernel, rows_grid, dim3(256), 0, s, S, L, scale);
    GemmArgs b{};
    b.M = L; b.N = dh; b.K = L;
    b.A = S; b.lda = L; b.transA = 0; b.lowerA = 1;
    b.B = V + off; b.ldb = ld; b.transB = 0;
    b.C = O + sq * L * ldo; b.ldc = ldo;
    b.alpha = 1.0f; b.beta = 0.0f; b.tri = 0;
    b.batch = heads; b.sA = L * L; b.sB = dh; b.sC = dh;
    if ((e = gemm_f32(b, s)) != hipSuccess) return e;
  }
  return hipGetLastError();
}

hipError_t silu_mul(const float* g, const float* u, int64_t n, float* y, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(silu_mul_kernel, dim3(grid_for(n)), dim3(256), 0, s, g, u, n, y);
  return hipGetLastError();
}

hipError_t to_f32(const void* x, int dtype, int64_t n, float* y, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(to_f32_kernel, dim3(grid_for(n)), dim3(256), 0, s, x, dtype, n, y);
  return hipGetLastError();
}

// ------------------------------------------------------------------ the block driver

namespace {

size_t up256(size_t b) { return (b + 255) & ~(size_t)255; }

// Layer i of the block (q, k, v, o, gate, up, down): output features and input features.
void layer_dims(const gptq_block_shape_t& sh, int i, int64_t& rows, int64_t& d) {
  rows = (i == 4 || i == 5) ? sh.inter : sh.hidden;
  d = i == 6 ? sh.inter : sh.hidden;
}

}  // namespace

BlockLayout block_layout(const gptq_block_shape_t& sh, const gptq_params_t& p) {
  BlockLayout L{};
  const int64_t n = sh.seqs * sh.seq_len, hd = sh.hidden, di = sh.inter, dm = std::max(hd, di);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += up256(bytes);
    return o;
  };
  const size_t act = (size_t)n * hd * 4;
  L.off_xf = take(act);
  L.off_xa = take(act);
  L.off_q = take(act);
  L.off_k = take(act);
  L.off_v = take(act);
  L.off_at = take(act);
  L.off_h1 = take(act);
  L.off_xm = take(act);
  L.off_g = take((size_t)n * di * 4);
  L.off_u = take((size_t)n * di * 4);
  L.off_s = take((size_t)sh.heads * sh.seq_len * sh.seq_len * 4);
  L.off_qk3 = take((size_t)2 * n * sh.heads * split3_pitch(hd / sh.heads) * 2);   // split Q and K
  L.off_wf = take((size_t)di * hd * 4);
  L.off_h = take((size_t)dm * dm * 4);
  L.off_uf = take((size_t)dm * dm * 4);
  L.off_xs = take((size_t)n * split3_pitch(dm) * 2);   // a stage input as fp16 [hi | hi | lo | 0]
  size_t w3 = 0;
  for (int i = 0; i < 7; ++i) {
    int64_t rows, d;
    layer_dims(sh, i, rows, d);
    w3 = std::max(w3, (size_t)rows * split3_pitch(d) * 2);
  }
  L.off_w3 = take(w3);                                  // a weight as fp16 [hi | lo | hi | 0]
  L.off_mx = take((size_t)(kAbsmaxParts + 1) * 4);
  L.off_h2 = take((size_t)4 * dm * dm * 4);             // 2 dm x 2 dm fp32
  L.hess_bytes = std::max(gptq_workspace_bytes(GPTQ_WS_HESSIAN, n, 2 * hd, nullptr),
                          gptq_workspace_bytes(GPTQ_WS_HESSIAN, n, 2 * di, nullptr));
  L.off_hw = take(L.hess_bytes);
  L.factor_bytes = gptq_workspace_bytes(GPTQ_WS_FACTOR, 0, dm, &p);
  L.off_fw = take(L.factor_bytes);
  L.quant_bytes = 0;
  for (int i = 0; i < 7; ++i) {
    int64_t rows, d;
    layer_dims(sh, i, rows, d);
    L.quant_bytes = std::max(L.quant_bytes, gptq_workspace_bytes(GPTQ_WS_QUANTIZE, rows, d, &p));
  }
  L.off_qw = take(L.quant_bytes);
  L.total = off;
  return L;
}

// True-sequential order (GPTQ tools page, "How it works", Step 9): q, k and v share the attention
// input; o's input is recomputed through the quantized q, k, v; gate and up share the MLP input,
// recomputed through the quantized o; down's input through the quantized gate and up. With
// true_sequential = 0 every input comes from the block with its original weights. The block output
// Y always runs through the quantized weights (the next block's input).
int quantize_block(const gptq_block_shape_t& sh, const void* X, int x_dtype, const gptq_params_t& p,
                   int true_sequential, const gptq_block_layer_t* layers, float* Y, float* const* hess, char* work,
                   int64_t* info, hipStream_t s) {
  const BlockLayout L = block_layout(sh, p);
  const int64_t n = sh.seqs * sh.seq_len, hd = sh.hidden, di = sh.inter;
  float* xf = reinterpret_cast<float*>(work + L.off_xf);
  float* xa = reinterpret_cast<float*>(work + L.off_xa);
  float* q = reinterpret_cast<float*>(work + L.off_q);
  float* k = reinterpret_cast<float*>(work + L.off_k);
  float* v = reinterpret_cast<float*>(work + L.off_v);
  float* at = reinterpret_cast<float*>(work + L.off_at);
  float* h1 = reinterpret_cast<float*>(work + L.off_h1);
  float* xm = reinterpret_cast<float*>(work + L.off_xm);
  float* gb = reinterpret_cast<float*>(work + L.off_g);
  float* ub = reinterpret_cast<float*>(work + L.off_u);
  float* S = reinterpret_cast<float*>(work + L.off_s);
  float* Wf = reinterpret_cast<float*>(work + L.off_wf);
  float* H = reinterpret_cast<float*>(work + L.off_h);
  float* U = reinterpret_cast<float*>(work + L.off_uf);
  const float eps = (float)sh.eps;
#define GPTQ_TRY(x)                                   \
  do {                                                \
    if ((x) != hipSuccess) return GPTQ_EHIP;          \
  } while (0)

  // H of the stage input (already split), then U, the order and the column loop of every layer
  // reading it
  auto stage = [&](int si, int64_t d, int first, int last) -> int {
    // H = 2 A^T A on the fp16 MFMA: H2 = 2 [hi | lo]^T [hi | lo] from the split input (its columns
    // d .. 3d - 1), folded
    int st;
    const _Float16* Xs = reinterpret_cast<const _Float16*>(work + L.off_xs) + d;
    float* H2 = reinterpret_cast<float*>(work + L.off_h2);
    // overwritten, not accumulated: the fold below reads H2 on and above its diagonal only
    if ((st = gptq_hessian_compute(H2, 2 * d, Xs, GPTQ_F16, n, split3_pitch(d), work + L.off_hw, L.hess_bytes,
                                   s)) != GPTQ_OK)
      return st;
    hipLaunchKernelGGL(fold_split_kernel, dim3(grid_for(d * d)), dim3(256), 0, s, H2, d, H);
    GPTQ_TRY(hipGetLastError());
    if (hess && hess[si]) GPTQ_TRY(hipMemcpyAsync(hess[si], H, (size_t)d * d * 4, hipMemcpyDeviceToDevice, s));
    int64_t piv = 0;
    st = gptq_factor(H, d, n, &p, U, layers[first].perm, work + L.off_fw, L.factor_bytes, &piv, s);
    if (st != GPTQ_OK) {
      info[0] = si;
      info[1] = piv;
      return st;
    }
    for (int i = first; i <= last; ++i) {
      int64_t rows, dd;
      layer_dims(sh, i, rows, dd);
      if (i != first && layers[i].perm != layers[first].perm)
        GPTQ_TRY(hipMemcpyAsync(layers[i].perm, layers[first].perm, (size_t)d * 4, hipMemcpyDeviceToDevice, s));
      st = gptq_quantize_layer(layers[i].W, layers[i].w_dtype, rows, d, d, U, layers[i].perm, &p, layers[i].codes,
                               layers[i].scales, layers[i].zeros, layers[i].g_idx, layers[i].loss, work + L.off_qw,
                               L.quant_bytes, s);
      if (st != GPTQ_OK) return st;
    }
    return GPTQ_OK;
  };
  // dense fp32 weights of layer i: its quantized values or its original ones
  auto weight = [&](int i, bool quantized) -> hipError_t {
    int64_t rows, d;
    layer_dims(sh, i, rows, d);
    if (!quantized) return to_f32(layers[i].W, layers[i].w_dtype, rows * d, Wf, s);
    const int64_t g = p.group_size <= 0 ? d : p.group_size;
    return dequantize(layers[i].codes, rows, d, layers[i].scales, layers[i].zeros, layers[i].g_idx, g, Wf, d, s);
  };
  // the current input A [n x d] as fp16 [hi | hi | lo | 0]
  auto split_input = [&](const float* A, int64_t d) -> hipError_t {
    return split3(A, n, d, d, 1.0f, 1, reinterpret_cast<_Float16*>(work + L.off_xs), s);
  };
  // out = A W_i^T (+ out when accumulate) for the split input A: W_i scaled by 2^k (max |2^k W_i| in
  // [2^14, 2^15), so its lo parts stay normal fp16) and split, one fp16 GEMM over 3d, alpha = 2^-k
  float* mx = reinterpret_cast<float*>(work + L.off_mx);
  auto project = [&](int i, bool quantized, float* out, bool accumulate) -> int {
    int64_t rows, d;
    layer_dims(sh, i, rows, d);
    GPTQ_TRY(weight(i, quantized));
    GPTQ_TRY(absmax(Wf, rows * d, mx + 1, mx, s));
    float wmax = 0.0f;
    GPTQ_TRY(hipMemcpyAsync(&wmax, mx, 4, hipMemcpyDeviceToHost, s));
    GPTQ_TRY(hipStreamSynchronize(s));
    int k = 0;
    if (wmax > 0.0f && std::isfinite(wmax)) k = std::min(100, std::max(-100, 14 - std::ilogb(wmax)));
    _Float16* W3 = reinterpret_cast<_Float16*>(work + L.off_w3);
    GPTQ_TRY(split3(Wf, rows, d, d, std::ldexp(1.0f, k), 0, W3, s));
    GemmF16 a{};
    a.M = n; a.N = rows; a.K = split3_pitch(d);
    a.A = reinterpret_cast<const _Float16*>(work + L.off_xs); a.lda = a.K;
    a.B = W3; a.ldb = a.K;
    a.C = out; a.ldc = rows;
    a.alpha = std::ldexp(1.0f, -k); a.beta = accumulate ? 1.0f : 0.0f;
    GPTQ_TRY(gemm_f16nt(a, s));
    return GPTQ_OK;
  };
  // one pass over the block; quantize: run each stage's solve before its layers are used
  auto pass = [&](bool quantized, bool quantize) -> int {
    int st;
    GPTQ_TRY(rmsnorm(xf, n, hd, hd, eps, xa, hd, s));
    GPTQ_TRY(split_input(xa, hd));
    if (quantize && (st = stage(0, hd, 0, 2)) != GPTQ_OK) return st;
    if ((st = project(0, quantized, q, false)) != GPTQ_OK) return st;
    if ((st = project(1, quantized, k, false)) != GPTQ_OK) return st;
    if ((st = project(2, quantized, v, false)) != GPTQ_OK) return st;
    GPTQ_TRY(causal_attention(q, k, v, sh.seqs, sh.seq_len, sh.heads, hd / sh.heads, hd, at, hd, S,
                              reinterpret_cast<_Float16*>(work + L.off_qk3), s));
    GPTQ_TRY(split_input(at, hd));
    if (quantize && (st = stage(1, hd, 3, 3)) != GPTQ_OK) return st;
    GPTQ_TRY(hipMemcpyAsync(h1, xf, (size_t)n * hd * 4, hipMemcpyDeviceToDevice, s));
    if ((st = project(3, quantized, h1, true)) != GPTQ_OK) return st;
    GPTQ_TRY(rmsnorm(h1, n, hd, hd, eps, xm, hd, s));
    GPTQ_TRY(split_input(xm, hd));
    if (quantize && (st = stage(2, hd, 4, 5)) != GPTQ_OK) return st;
    if ((st = project(4, quantized, gb, false)) != GPTQ_OK) return st;
    if ((st = project(5, quantized, ub, false)) != GPTQ_OK) return st;
    GPTQ_TRY(silu_mul(gb, ub, n * di, gb, s));
    GPTQ_TRY(split_input(gb, di));
    if (quantize && (st = stage(3, di, 6, 6)) != GPTQ_OK) return st;
    GPTQ_TRY(hipMemcpyAsync(Y, h1, (size_t)n * hd * 4, hipMemcpyDeviceToDevice, s));
    if ((st = project(6, true, Y, true)) != GPTQ_OK) return st;
    return GPTQ_OK;
  };
#undef GPTQ_TRY
  info[0] = -1;
  info[1] = 0;
  if (to_f32(X, x_dtype, n * hd, xf, s) != hipSuccess) return GPTQ_EHIP;
  int st = pass(true_sequential != 0, true);
  if (st == GPTQ_OK && !true_sequential) st = pass(true, false);
  return st;
}

}  // namespace gptq
