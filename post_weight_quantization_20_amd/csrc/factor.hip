// Damping, act-order and the upper Cholesky factor U of the damped inverse Hessian (Hhat^-1 = U^T U).
//
// GPTQ tools page, "How it works", Step 4 (damping: a small multiple of the mean diagonal is added
// to the diagonal), "Optional refinements" (act-order: columns by descending diag(H)), and Step 6
// (the Cholesky factor of the inverse Hessian is computed once; its rows give every step's update).
//
// Route. With J the exchange matrix, if J Hhat J = L L^T (lower Cholesky) then Hhat = R R^T with
// R = J L J upper, and U = R^-1 = J L^-1 J. So the damped, permuted Hessian is gathered already
// reversed, factored by a blocked right-looking Cholesky, inverted in place by a blocked
// right-looking triangular inverse, and rotated back by 180 degrees. This takes 2/3 d^3 flops and
// never forms Hhat^-1 (the page's sketch takes the Cholesky factor of Hhat, forms the inverse from it
// and factors that again, 4/3 d^3 flops; both give the same U in exact arithmetic).
//
// Blocking (nb = 128): per diagonal block one workgroup factors the block in LDS and replaces it
// by the inverse of its Cholesky factor; every other product (panel solve, symmetric trailing
// update, the triangular-inverse products) is an fp32 MFMA GEMM on the whole device.
#include "common.hpp"

namespace gptq {
namespace {

constexpr int NB = 128;
constexpr int NBP = NB + 1;  // LDS row length (odd: column walks do not collide on banks)

struct FactorWork {
  double* lam;     // damping added to the diagonal
  int64_t* info;   // 0, or the 1-based index of the first non-positive pivot
  int* status;     // 1 when mean(diag H) is not positive and finite
  float* keys;     // diag(H), the act-order sort key
};

// mean(diag(H)) / n * damp, in float64 and a fixed summation order; also copies diag(H).
__global__ __launch_bounds__(1024) void diag_stats_kernel(const float* __restrict__ H, int64_t d, int64_t n,
                                                          double damp, FactorWork w) {
  __shared__ double part[1024];
  double acc = 0.0;
  for (int64_t i = threadIdx.x; i < d; i += 1024) {
    const float h = H[i * d + i];
    w.keys[i] = h;
    acc += (double)h;
  }
  part[threadIdx.x] = acc;
  __syncthreads();
  for (int s = 512; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) part[threadIdx.x] += part[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double mean = part[0] / (double)d / (double)n;
    const bool ok = mean > 0.0 && mean < 1.0e300;
    *w.status = ok ? 0 : 1;
    *w.lam = ok ? damp * mean : 0.0;
    *w.info = 0;
  }
}

// perm[rank(i)] = i with rank = number of keys that sort before key i: larger keys first, equal
// keys by lower index first (a stable descending sort). NaN keys sort last.
__global__ __launch_bounds__(256) void rank_perm_kernel(const float* __restrict__ keys, int64_t d,
                                                        int32_t* __restrict__ perm) {
  __shared__ float tile[2048];
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  float ki = i < d ? keys[i] : 0.0f;
  if (ki != ki) ki = -INFINITY;
  int64_t rank = 0;
  for (int64_t t0 = 0; t0 < d; t0 += 2048) {
    const int64_t cnt = min<int64_t>(2048, d - t0);
    __syncthreads();
    for (int e = threadIdx.x; e < cnt; e += 256) {
      float v = keys[t0 + e];
      tile[e] = (v != v) ? -INFINITY : v;
    }
    __syncthreads();
    if (i < d) {
      for (int e = 0; e < cnt; ++e) {
        const float kj = tile[e];
        const int64_t j = t0 + e;
        rank += (kj > ki) || (kj == ki && j < i);
      }
    }
  }
  if (i < d) perm[rank] = (int32_t)i;
}

__global__ void iota_kernel(int32_t* perm, int64_t d) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < d) perm[i] = (int32_t)i;
}

// A[i][j] (j <= i) = Hhat[p(i)][p(j)], p(i) = perm[d-1-i]: the damped, normalised Hessian in
// processing order, reversed. H's upper triangle is authoritative.
__global__ __launch_bounds__(256) void gather_kernel(const float* __restrict__ H, int64_t d, int64_t n,
                                                     const int32_t* __restrict__ perm, FactorWork w,
                                                     float* __restrict__ A) {
  const int64_t i = blockIdx.x;
  const int64_t pi = perm[d - 1 - i];
  const double lam = *w.lam;
  const double inv_n = 1.0 / (double)n;
  for (int64_t j = threadIdx.x; j <= i; j += 256) {
    const int64_t pj = perm[d - 1 - j];
    const int64_t r = min(pi, pj), c = max(pi, pj);
    double v = (double)H[r * d + c] * inv_n;
    if (pi == pj) v += lam;
    A[i * d + j] = (float)v;
  }
}

// Factors the diagonal block at (k0, k0) in LDS (A = L L^T, lower) and replaces the whole block in A
// by the inverse of L (lower triangle; zeros above). A first non-positive pivot is recorded in info
// and replaced by 1 so the remaining arithmetic stays finite.
__global__ __launch_bounds__(256) void chol_diag_kernel(float* __restrict__ A, int64_t d, int64_t k0, int nb,
                                                        int64_t* __restrict__ info) {
  extern __shared__ float sm[];
  float* L = sm;              // [NB][NBP]
  float* X = sm + NB * NBP;   // [NB][NBP]
  __shared__ float dia[NB];
  __shared__ float piv;
  const int tid = threadIdx.x;
  for (int e = tid; e < NB * NB; e += 256) {
    const int r = e / NB, c = e % NB;
    L[r * NBP + c] = (r < nb && c <= r) ? A[(k0 + r) * d + k0 + c] : 0.0f;
    X[r * NBP + c] = (r == c) ? 1.0f : 0.0f;
  }
  __syncthreads();
  // Right-looking Cholesky. Column j is read unscaled in step j (products divided by the pivot)
  // and scaled in step j + 1, so each step needs two barriers.
  for (int j = 0; j < nb; ++j) {
    if (tid == 0) {
      float p = L[j * NBP + j];
      if (!(p > 0.0f)) {
        if (*info == 0) *info = k0 + j + 1;
        p = 1.0f;
      }
      piv = p;
      dia[j] = sqrtf(p);
    }
    __syncthreads();
    const float inv_p = 1.0f / piv;
    if (j > 0) {
      const float dprev = dia[j - 1];
      for (int i = j + tid; i < nb; i += 256) L[i * NBP + (j - 1)] /= dprev;
    }
    // trailing update: L[i][c] -= L[i][j] L[c][j] / p for j < c <= i
    const int m = nb - j - 1;
    const int cnt = m * (m + 1) / 2;
    for (int e = tid; e < cnt; e += 256) {
      int ii = (int)((sqrtf(8.0f * e + 1.0f) - 1.0f) * 0.5f);
      while ((ii + 1) * (ii + 2) / 2 <= e) ++ii;
      while (ii * (ii + 1) / 2 > e) --ii;
      const int cc = e - ii * (ii + 1) / 2;
      const int i = j + 1 + ii, c = j + 1 + cc;
      L[i * NBP + c] -= L[i * NBP + j] * L[c * NBP + j] * inv_p;
    }
    __syncthreads();
  }
  for (int j = tid; j < nb; j += 256) L[j * NBP + j] = dia[j];
  __syncthreads();
  // Inverse of L by forward elimination on [L | I], right-looking: when row j is reached it holds
  // e_j - sum_{t<j} L[j][t] X[t]; dividing by L[j][j] finishes it (done one step late, like above).
  for (int j = 0; j < nb; ++j) {
    const float inv_l = 1.0f / L[j * NBP + j];
    if (j > 0) {
      const float inv_prev = 1.0f / L[(j - 1) * NBP + (j - 1)];
      for (int c = tid; c <= j - 1; c += 256) X[(j - 1) * NBP + c] *= inv_prev;
    }
    const int rows_below = nb - j - 1, cols = j + 1;
    for (int e = tid; e < rows_below * cols; e += 256) {
      const int i = j + 1 + e / cols, c = e % cols;
      X[i * NBP + c] -= L[i * NBP + j] * X[j * NBP + c] * inv_l;
    }
    __syncthreads();
  }
  if (nb > 0) {
    const float inv_last = 1.0f / L[(nb - 1) * NBP + (nb - 1)];
    for (int c = tid; c < nb; c += 256) X[(nb - 1) * NBP + c] *= inv_last;
  }
  __syncthreads();
  for (int e = tid; e < NB * NB; e += 256) {
    const int r = e / NB, c = e % NB;
    if (r < nb && c < nb) A[(k0 + r) * d + k0 + c] = (c <= r) ? X[r * NBP + c] : 0.0f;
  }
}

// 180-degree rotation in place: the lower triangle of the inverted reversed factor becomes U's
// upper triangle; U's strict lower triangle is set to zero.
__global__ __launch_bounds__(256) void flip_kernel(float* __restrict__ A, int64_t d) {
  const int64_t i = blockIdx.x;
  for (int64_t j = threadIdx.x; j < i; j += 256) {
    const float v = A[i * d + j];
    A[(d - 1 - i) * d + (d - 1 - j)] = v;
    A[i * d + j] = 0.0f;
  }
  if (threadIdx.x == 0 && i < d - 1 - i) {
    const float a = A[i * d + i], b = A[(d - 1 - i) * d + (d - 1 - i)];
    A[i * d + i] = b;
    A[(d - 1 - i) * d + (d - 1 - i)] = a;
  }
}

size_t chol_smem() { return (size_t)2 * NB * NBP * sizeof(float); }

}  // namespace

size_t factor_workspace_bytes(int64_t d) { return 256 + (size_t)d * sizeof(float); }

// Returns hipSuccess after queueing everything; *status_out / *info_out are device addresses of the
// status word and pivot index (read by the caller after a stream synchronisation).
hipError_t factor(const float* H, int64_t d, int64_t n, double damp, int act_order, float* U, int32_t* perm,
                  void* work, hipStream_t s, int** status_dev, int64_t** info_dev) {
  char* wb = static_cast<char*>(work);
  FactorWork w;
  w.lam = reinterpret_cast<double*>(wb);
  w.info = reinterpret_cast<int64_t*>(wb + 8);
  w.status = reinterpret_cast<int*>(wb + 16);
  w.keys = reinterpret_cast<float*>(wb + 256);
  *status_dev = w.status;
  *info_dev = w.info;

  hipLaunchKernelGGL(diag_stats_kernel, dim3(1), dim3(1024), 0, s, H, d, n, damp, w);
  if (act_order)
    hipLaunchKernelGGL(rank_perm_kernel, dim3((unsigned)((d + 255) / 256)), dim3(256), 0, s, w.keys, d, perm);
  else
    hipLaunchKernelGGL(iota_kernel, dim3((unsigned)((d + 255) / 256)), dim3(256), 0, s, perm, d);
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)d), dim3(256), 0, s, H, d, n, perm, w, U);

  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute((const void*)chol_diag_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                        (int)chol_smem());
    attr = true;
  }
  hipError_t e;
  const int64_t nblk = (d + NB - 1) / NB;
  // blocked right-looking Cholesky of the reversed matrix; diagonal blocks end up inverted
  for (int64_t k = 0; k < nblk; ++k) {
    const int64_t k0 = k * NB, k1 = std::min(d, k0 + NB), kb = k1 - k0;
    hipLaunchKernelGGL(chol_diag_kernel, dim3(1), dim3(256), chol_smem(), s, U, d, k0, (int)kb, w.info);
    if (k1 < d) {
      GemmArgs t{};  // panel solve: P <- P L_kk^-T
      t.M = d - k1; t.N = kb; t.K = kb;
      t.A = U + k1 * d + k0; t.lda = d; t.transA = 0;
      t.B = U + k0 * d + k0; t.ldb = d; t.transB = 1;
      t.C = U + k1 * d + k0; t.ldc = d;
      t.alpha = 1.0f; t.beta = 0.0f; t.tri = 0;
      if ((e = gemm_f32(t, s)) != hipSuccess) return e;
      GemmArgs u{};  // trailing update: A22 -= P P^T (lower part)
      u.M = d - k1; u.N = d - k1; u.K = kb;
      u.A = U + k1 * d + k0; u.lda = d; u.transA = 0;
      u.B = U + k1 * d + k0; u.ldb = d; u.transB = 1;
      u.C = U + k1 * d + k1; u.ldc = d;
      u.alpha = -1.0f; u.beta = 1.0f; u.tri = 1;
      if ((e = gemm_f32(u, s)) != hipSuccess) return e;
    }
  }
  // blocked right-looking inverse of the lower factor, in place (diagonal blocks already inverted)
  for (int64_t j = 0; j < nblk; ++j) {
    const int64_t j0 = j * NB, j1 = std::min(d, j0 + NB), jb = j1 - j0;
    if (j0 > 0) {
      GemmArgs r{};  // row panel: R <- -X_jj R
      r.M = jb; r.N = j0; r.K = jb;
      r.A = U + j0 * d + j0; r.lda = d; r.transA = 0;
      r.B = U + j0 * d; r.ldb = d; r.transB = 0;
      r.C = U + j0 * d; r.ldc = d;
      r.alpha = -1.0f; r.beta = 0.0f; r.tri = 0;
      if ((e = gemm_f32(r, s)) != hipSuccess) return e;
      if (j1 < d) {
        GemmArgs q{};  // rectangle: A[j1:, :j0] += L[j1:, j] R
        q.M = d - j1; q.N = j0; q.K = jb;
        q.A = U + j1 * d + j0; q.lda = d; q.transA = 0;
        q.B = U + j0 * d; q.ldb = d; q.transB = 0;
        q.C = U + j1 * d; q.ldc = d;
        q.alpha = 1.0f; q.beta = 1.0f; q.tri = 0;
        if ((e = gemm_f32(q, s)) != hipSuccess) return e;
      }
    }
    if (j1 < d) {
      GemmArgs c{};  // column panel: L[j1:, j] <- L[j1:, j] X_jj
      c.M = d - j1; c.N = jb; c.K = jb;
      c.A = U + j1 * d + j0; c.lda = d; c.transA = 0;
      c.B = U + j0 * d + j0; c.ldb = d; c.transB = 0;
      c.C = U + j1 * d + j0; c.ldc = d;
      c.alpha = 1.0f; c.beta = 0.0f; c.tri = 0;
      if ((e = gemm_f32(c, s)) != hipSuccess) return e;
    }
  }
  hipLaunchKernelGGL(flip_kernel, dim3((unsigned)d), dim3(256), 0, s, U, d);
  return hipGetLastError();
}

}  // namespace gptq
