/*
 * GPTQ single-layer solver for AMD Instinct MI355X (gfx950): C ABI.
 *
 * The solver quantizes one linear layer's weights W (rows x d, d = input features) to low-bit
 * integer codes with a scale and zero point per group, pushing each column's rounding error onto the
 * columns not yet quantized through the Cholesky factor of the inverse Hessian of the layer's
 * calibration inputs X (tokens x d). The four calls below are its steps, in order:
 *
 *   gptq_hessian_accumulate  H += 2 X_c^T X_c for each token chunk X_c (gptq_hessian_compute:
 *                            H = 2 X_c^T X_c, for the first chunk)
 *   gptq_factor              damping, optional act-order, U = upper Cholesky factor of Hhat^-1
 *   gptq_quantize_layer      the column loop with lazy block updates; codes, scales, zeros, loss
 *   gptq_pack                eight 4-bit codes per 32-bit word (four 8-bit ones)
 *   gptq_pack_dense          the codes as one dense bit stream per row
 *   gptq_pack_ordered        the codes in a column order (act-order layers stored in processing order)
 *   gptq_permute_columns     inputs gathered by the same order
 *
 * and one call that uses the stored layer:
 *
 *   gptq_dequant_gemm        y = x W^T for a few input rows, read straight from the packed codes
 *
 * Sources (web pages on GPTQ): the GPTQ tools page at ozercemkelahmet.com ("How it works",
 * Steps 3-8, "Optional refinements", "A minimal Python sketch", "Memory arithmetic"); "GPTQ
 * Quantization: Complete Technical Guide" (notes.jayaprakash.net; "Quantization Equation",
 * "Computing the Hessian", "Damping Factor", "Configuration Deep Dive"); "Paper breakdown: GPTQ"
 * (ai360xpert.com; "How It Works", lazy batching); "What Is GPTQ?" (ai-tldr.dev; "How it works",
 * Step 3, groups).
 *
 * Conventions for every call:
 *   - Matrices are row-major. Pointers named as device memory must be device memory of the current
 *     HIP device; the caller allocates and owns every buffer and the library allocates no device
 *     memory. The only state it keeps: on first use on a device it creates two helper streams and a
 *     few events there (kept until the process ends), on which parts of a call run concurrently;
 *     and one static device array, the workspace of gptq_factor_noalloc.
 *   - `stream` is a hipStream_t (NULL: the default stream). Work is queued on it and the call returns
 *     without waiting, except gptq_factor, which waits once for its own work (see there). Work a call
 *     places on the helper streams starts after the work queued on `stream` before the call and
 *     ends before the call's later work on `stream`, so the call is ordered on `stream` as a whole.
 *   - Arguments are checked on the host before anything is queued. A rejected call returns a negative
 *     status and has no effect. HIP launch failures return GPTQ_EHIP.
 *   - Calls that share no output buffer may run concurrently on different streams.
 */
#ifndef GPTQ_H
#define GPTQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t gptq_status_t;

enum {
  GPTQ_OK = 0,
  GPTQ_EINVAL = -1,       /* invalid argument (null pointer, bad size, inconsistent settings)   */
  GPTQ_ENOTPD = -2,       /* damped Hessian not positive definite (see gptq_factor's info)      */
  GPTQ_EUNSUPPORTED = -3, /* a setting this library does not implement (e.g. block_size > 128)  */
  GPTQ_EHIP = -4,         /* a HIP runtime call or kernel launch failed                         */
  GPTQ_ENOMEM = -5        /* the workspace passed is smaller than gptq_workspace_bytes asks     */
};

/* Element types of W and X. */
enum { GPTQ_F32 = 0, GPTQ_F16 = 1, GPTQ_BF16 = 2 };

/* Storage layouts of packed codes (gptq_dequant_gemm's `layout`). */
enum {
  GPTQ_LAYOUT_FIELDS = 0, /* gptq_pack: a nibble per code up to 4 bits (8 per word), a byte above    */
  GPTQ_LAYOUT_DENSE = 1   /* gptq_pack_dense: exactly `bits` bits per code in one bit stream per row */
};

/* Workspace kinds for gptq_workspace_bytes. */
enum { GPTQ_WS_HESSIAN = 0, GPTQ_WS_FACTOR = 1, GPTQ_WS_QUANTIZE = 2 };

/* Quantization settings (the configuration surface of the Technical Guide's AutoGPTQ example:
 * bits, group_size, desc_act, damp_percent; the lazy-batch block size of the tools page, Step 7). */
typedef struct {
  int32_t bits;          /* code width, 2..8; codes are unsigned in [0, 2^bits - 1]             */
  int32_t group_size;    /* columns per group (>= 2); <= 0: one group per row. Groups and blocks
                            must nest: block_size % group_size == 0 or group_size % block_size == 0.
                            A group size of 1 is rejected (Technical Guide, "Don'ts").          */
  int32_t block_size;    /* lazy-batch width B, 1..128 (tools page, Step 7: "often 128")        */
  int32_t act_order;     /* 1: process columns by descending diag(H) (tools page, Act-order)     */
  int32_t sym;           /* 0: asymmetric min/max grid, zero = round(-wmin / scale); 1: symmetric
                            grid (tools page, "Optional refinements"): scale = max(2 max|w|, 1e-8)
                            / maxq and zero = 2^(bits-1), the middle code, so value = scale x
                            (code - zero) spans the Technical Guide's signed range [-8, 7] steps
                            at 4 bits. Codes stay unsigned in [0, 2^bits - 1].                  */
  int32_t static_groups; /* 0: a group's grid is taken from the current, error-updated weights
                            when the loop reaches the group's first column (groups are g
                            consecutive processing positions); 1: every grid is fixed before the
                            loop from the original weights of g consecutive original columns,
                            each column uses its original group's grid, and g_idx = k / g also
                            with act-order (the Technical Guide's static_groups setting).        */
  int32_t compact_meta;  /* 1: each grid is what a 16-bit scale and a zero of the code width store
                            (tools page, "Memory arithmetic"), and the loop quantizes with exactly
                            that: the scale rounded to the nearest float16 (the smallest positive
                            float16 if it would round to zero), the zero clamped to [0, maxq].
                            The fp32 scales and int32 zeros written then convert to that storage
                            without loss.                                                      */
  double damp;           /* relative damping >= 0: lambda = damp * mean(diag(H / n)) (Step 4)     */
} gptq_params_t;

/*
 * H += 2 * X^T X over one chunk of calibration tokens (GPTQ tools page, "How it works", Step 3;
 * Technical Guide, "Computing the Hessian": a sum of outer products of the layer inputs).
 *
 *   H      device float[d * d]. Accumulated in place; zero it before the first chunk. Only the
 *          upper triangle (i <= j) is authoritative; entries below the diagonal are left as they
 *          were, except inside 256 x 256 diagonal tiles, where they may take their part of the sum.
 *   d      number of input features, >= 1.
 *   X      device array [n_tok x ld_x] of x_dtype (GPTQ_F32, GPTQ_F16 or GPTQ_BF16), token-major:
 *          row t holds the d features of token t. Not modified. May be NULL when n_tok == 0.
 *   n_tok  tokens in this chunk, >= 0 (0: nothing is queued).
 *   ld_x   row pitch of X in elements, >= d.
 *   work   device workspace of work_bytes bytes, or NULL. With at least
 *          gptq_workspace_bytes(GPTQ_WS_HESSIAN, n_tok, d, NULL) bytes the token range is split
 *          across more workgroups (partial sums are added in token order); with less (or NULL) it
 *          is not split, which sums in another order (same float32 error bound) and may be slower.
 *          The workspace must not be shared with a concurrent call.
 * fp16 / bf16 products are exact in fp32; sums are fp32. The result does not depend on scheduling.
 */
gptq_status_t gptq_hessian_accumulate(float *H, int64_t d, const void *X, int32_t x_dtype, int64_t n_tok,
                                      int64_t ld_x, void *work, size_t work_bytes, void *stream);

/*
 * H = 2 * X^T X over one chunk of calibration tokens: gptq_hessian_accumulate for the first chunk,
 * without zeroing H first (the same source passages). Same arguments and errors as
 * gptq_hessian_accumulate. H's upper triangle (i <= j) is overwritten and H is not read; entries
 * below the diagonal are written inside 256 x 256 diagonal tiles only (their part of the sum, or
 * zero). With n_tok == 0 the whole of H is set to zero. The result is bit for bit that of zeroing H
 * and calling gptq_hessian_accumulate with the same chunk and workspace.
 */
gptq_status_t gptq_hessian_compute(float *H, int64_t d, const void *X, int32_t x_dtype, int64_t n_tok,
                                   int64_t ld_x, void *work, size_t work_bytes, void *stream);

/*
 * Damping, processing order and the upper Cholesky factor of the damped inverse Hessian
 * (GPTQ tools page, "How it works", Steps 4 and 6; "Optional refinements", Act-order).
 *
 *   H        device float[d * d], the accumulated sum of gptq_hessian_accumulate (upper triangle
 *            read). Not modified, unless U == H.
 *   n_total  number of tokens summed into H (> 0); Hhat = H / n_total + lambda I with
 *            lambda = p->damp * mean(diag(H / n_total)).
 *   p        settings; reads damp, act_order, sym, static_groups.
 *   U        device float[d * d], output: upper-triangular U with Hhat_perm^-1 = U^T U, in
 *            processing order (row/column j is original column perm[j]); zeros below the diagonal.
 *            Either U == H (the factor overwrites H in place, with no second d x d buffer) or the
 *            two do not overlap; a partial overlap is GPTQ_EINVAL.
 *   perm     device int32[d], output: the processing order. Identity without act-order; with it,
 *            columns by descending diag(H), equal values by lower index first.
 *   work     device workspace of at least gptq_workspace_bytes(GPTQ_WS_FACTOR, 0, d, p) bytes.
 *   info     host int64 output: 0 on success; k > 0 when the k-th pivot (1-based, in the reversed
 *            order the factorization runs in) was not positive (U is then unspecified).
 * This call waits for the stream once, to read the pivot check. Returns GPTQ_ENOTPD when info != 0
 * (damping "helps but does not fix" a rank-deficient Hessian: retry with a larger damp), GPTQ_EINVAL
 * when mean(diag(H)) is not positive and finite.
 */
gptq_status_t gptq_factor(const float *H, int64_t d, int64_t n_total, const gptq_params_t *p, float *U,
                          int32_t *perm, void *work, size_t work_bytes, int64_t *info, void *stream);

/*
 * gptq_factor for callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation. Same arguments, results and errors as
 * gptq_factor, without `work`: its workspace is a static device array inside the library (about
 * 25 MB, held on each device the library runs on until the process ends), and every launch goes to
 * `stream` (no helper stream or event is created). The call allocates nothing; the caller still
 * passes H, U and perm (U == H allowed, as for gptq_factor).
 *
 *   d  at most GPTQ_FACTOR_NOALLOC_MAX_D; larger d returns GPTQ_EUNSUPPORTED.
 *
 * All calls on one device share that device's array, and each call overwrites it: calls that
 * overlap on one device (on different streams or host threads) race. Like gptq_factor, the call
 * waits for the stream once to read the pivot check.
 */
#define GPTQ_FACTOR_NOALLOC_MAX_D 12288
gptq_status_t gptq_factor_noalloc(const float *H, int64_t d, int64_t n_total, const gptq_params_t *p, float *U,
                                  int32_t *perm, int64_t *info, void *stream);

/*
 * The GPTQ column loop for one layer (GPTQ tools page, "How it works", Steps 5, 7 and 8; the
 * Technical Guide's "Quantization Equation" grid; "What Is GPTQ?", Step 3 groups).
 *
 *   W       device array [rows x ld_w] of w_dtype (GPTQ_F32, GPTQ_F16 or GPTQ_BF16), original column
 *           order. Not modified.
 *   rows    output features, >= 0 (0: only g_idx is written and loss is set to 0).
 *   d       input features, >= 1; ld_w >= d.
 *   U, perm from gptq_factor with the same d and act_order.
 *   p       settings; reads bits, group_size, block_size, sym, static_groups.
 *   codes   device uint8[rows * d], output: codes in [0, 2^bits - 1], original column order.
 *   scales  device float[rows * ngroups], zeros device int32[rows * ngroups], output, with
 *           ngroups = ceil(d / g) and g = group_size (d when group_size <= 0). Group j of a row
 *           covers processing positions [j g, (j+1) g), or original columns [j g, (j+1) g) with
 *           static_groups; dequantized value = scale * (code - zero).
 *   g_idx   device int32[d], output: the group of each original column.
 *   loss    device double[1], output: the sum over rows and columns of err^2, where err is a
 *           column's rounding error divided by the factor's diagonal entry; it equals
 *           sum_r (W - Q)_r Hhat (W - Q)_r^T (the damped layer objective, tools page Step 2).
 *   work    device workspace of at least gptq_workspace_bytes(GPTQ_WS_QUANTIZE, rows, d, p) bytes.
 * Rounding is to nearest, ties to even; the rounding ratios are taken in fp32 with correctly rounded
 * division. Rows are independent: splitting W by rows over calls gives the same results.
 */
gptq_status_t gptq_quantize_layer(const void *W, int32_t w_dtype, int64_t rows, int64_t d, int64_t ld_w,
                                  const float *U, const int32_t *perm, const gptq_params_t *p, uint8_t *codes,
                                  float *scales, int32_t *zeros, int32_t *g_idx, double *loss, void *work,
                                  size_t work_bytes, void *stream);

/*
 * gptq_quantize_layer with a breakdown of where its device time goes (measurement: the same work
 * and results, plus events recorded between its launches). Same arguments, plus:
 *   part_ms  host double[3], output: device milliseconds of the column-loop kernels (the in-block
 *            chain with the lazy updates inside each super-block of up to 512 columns), of the lazy
 *            products that carry each super-block's errors to the later columns (fp32 MFMA GEMMs),
 *            and of the rest (working copy, indices, un-permute, loss). NULL is GPTQ_EINVAL.
 * Unlike gptq_quantize_layer it waits for the stream before returning.
 */
gptq_status_t gptq_quantize_layer_timed(const void *W, int32_t w_dtype, int64_t rows, int64_t d, int64_t ld_w,
                                        const float *U, const int32_t *perm, const gptq_params_t *p, uint8_t *codes,
                                        float *scales, int32_t *zeros, int32_t *g_idx, double *loss, void *work,
                                        size_t work_bytes, double *part_ms, void *stream);

/*
 * Packs codes in fixed fields along the columns (GPTQ tools page, "How it works", Step 8: eight 4-bit
 * codes per 32-bit word): a nibble per code for bits 1..4, a byte per code for bits 5..8.
 *
 *   codes   device uint8[rows * d]; every code must be < 2^bits (bits above the field are dropped).
 *   rows    >= 0; d >= 8 and a multiple of 8; bits in 1..8 (3-bit codes also take a nibble).
 *   packed  device int32[rows * d * f / 32], output, f = 4 or 8: bits f t .. f t + f - 1 of word k of
 *           a row hold column (32 / f) k + t.
 */
gptq_status_t gptq_pack(const uint8_t *codes, int64_t rows, int64_t d, int32_t bits, int32_t *packed,
                        void *stream);

/*
 * Packs codes as one dense bit stream per row, exactly `bits` bits per code, so 3-bit codes take 3
 * bits, not a nibble (the tools page's "Memory arithmetic": storage follows the bit width). At 4 and
 * 8 bits the words equal gptq_pack's.
 *
 *   codes   device uint8[rows * d]; every code must be < 2^bits (higher bits are dropped).
 *   rows    >= 0; d >= 1 with d * bits a multiple of 32; bits in 1..8.
 *   packed  device int32[rows * d * bits / 32], output: code k of a row occupies stream bits
 *           bits k .. bits k + bits - 1, and stream bit t is bit t % 32 of word t / 32 of the row.
 */
gptq_status_t gptq_pack_dense(const uint8_t *codes, int64_t rows, int64_t d, int32_t bits, int32_t *packed,
                              void *stream);

/*
 * Packs the codes in a given column order, in gptq_pack's field layout: column j of the output is
 * column order[j] of the codes. With order = gptq_factor's perm (the act-order processing order), a
 * group's columns are contiguous again (group j / g), so gptq_dequant_gemm can take its fast kernels
 * with g_idx = NULL on inputs gathered by the same order (gptq_permute_columns). The product is the
 * same sum taken in another order. This is the act-order trade-off of the tools page ("Optional
 * refinements"; What Is GPTQ, kernel speed) paid once at storage time instead of in every product.
 *
 *   codes   device uint8[rows * d], original column order (gptq_quantize_layer's codes).
 *   rows    >= 0; d >= 8 and a multiple of 8; bits in 1..8.
 *   order   device int32[d], a permutation of 0..d-1 (values outside [0, d) are clamped into it).
 *   packed  device int32[rows * d * f / 32], output, f = 4 for bits <= 4 and 8 above.
 */
gptq_status_t gptq_pack_ordered(const uint8_t *codes, int64_t rows, int64_t d, int32_t bits, const int32_t *order,
                                int32_t *packed, void *stream);

/*
 * Gathers the columns of a row-major matrix: out[i][j] = in[i][order[j]] (the layer inputs in the
 * order of codes packed by gptq_pack_ordered).
 *
 *   in      device array [m x ld_in] of dtype (GPTQ_F32, GPTQ_F16 or GPTQ_BF16). Not modified.
 *   m       rows, >= 0 (0: nothing is queued); d columns, >= 1; ld_in, ld_out >= d.
 *   order   device int32[d] (values outside [0, d) are clamped into it).
 *   out     device array [m x ld_out] of dtype, output; must not overlap `in`.
 */
gptq_status_t gptq_permute_columns(const void *in, int32_t dtype, int64_t m, int64_t d, int64_t ld_in,
                                   const int32_t *order, void *out, int64_t ld_out, void *stream);

/*
 * The stored layer at inference: y = x W^T for a few rows of inputs x, with W expanded from the packed
 * codes, scales and zeros inside the kernel (GPTQ tools page, "How it works", Step 8: a fused kernel
 * unpacks, scales and multiplies; "What Is GPTQ?", "How it works", Step 3: each group is expanded
 * back to higher precision just in time for the product). Small-batch products like this are bound
 * by reading the weights, about half a byte per weight here.
 *
 *   x       device array [m x ld_x] of x_dtype (GPTQ_F32, GPTQ_F16 or GPTQ_BF16): one row per token,
 *           d features each. Not modified.
 *   m       input rows, >= 0 (0: nothing is queued). Rows are taken eight at a time, and each group
 *           of eight reads the codes once.
 *   ld_x    row pitch of x in elements, >= d.
 *   packed  device int32 codes of rows x d weights in `layout`: GPTQ_LAYOUT_FIELDS is gptq_pack's
 *           (rows * d / 8 words of nibbles for bits <= 4, rows * d / 4 words of bytes above),
 *           GPTQ_LAYOUT_DENSE is gptq_pack_dense's (rows * d * bits / 32 words; d * bits must be
 *           a multiple of 32). Not modified.
 *   bits    the code width, 1..8.
 *   layout  GPTQ_LAYOUT_FIELDS or GPTQ_LAYOUT_DENSE.
 *   scales  device float[rows * ngroups] and zeros device int32[rows * ngroups], as
 *           gptq_quantize_layer writes them, with ngroups = ceil(d / g) and g = group_size (d when
 *           group_size <= 0).
 *   g_idx   device int32[d], the group of each column (gptq_quantize_layer's g_idx, needed after
 *           act-order), or NULL when column k is in group k / g. Entries outside [0, ngroups) are
 *           clamped into it.
 *   rows    weight rows (outputs), >= 0 (0: nothing is queued); d input columns, >= 8, a multiple
 *           of 8.
 *   y       device float[m x ld_y], output, ld_y >= rows: y[i, r] = sum_k x[i, k] W[r, k] with
 *           W[r, k] = scales[r, G] * (code[r, k] - zeros[r, G]) and G the group of column k.
 * Products and sums are fp32 (fp16 x times a code is exact in fp32). Faster kernels run for nibble
 * fields when x is fp16, g_idx is NULL, g is a multiple of 32 or at least d, d is a multiple of 32,
 * and the rows of x and the codes are 16-byte aligned (for 3 or more input rows also g a multiple of
 * 128 and d of 128); otherwise a general one does. Results do not depend on scheduling.
 */
gptq_status_t gptq_dequant_gemm(const void *x, int32_t x_dtype, int64_t m, int64_t ld_x, const int32_t *packed,
                                int32_t bits, int32_t layout, const float *scales, const int32_t *zeros,
                                const int32_t *g_idx, int64_t rows, int64_t d, int32_t group_size, float *y,
                                int64_t ld_y, void *stream);

/*
 * One pre-norm decoder block for gptq_quantize_block. The pages fix the order in which a block's
 * layers are solved but not the block itself; this one is RMSNorm -> multi-head causal
 * self-attention (q, k, v, o; no positional rotation) -> residual -> RMSNorm -> SiLU-gated MLP
 * (gate, up, down) -> residual, with no learned norm weights.
 */
typedef struct {
  int64_t hidden;   /* model width, >= 8; q, k, v, o are hidden x hidden                          */
  int64_t heads;    /* attention heads, 1..65535, dividing hidden; heads * seq_len <= 2^31        */
  int64_t inter;    /* MLP width, >= 8; gate and up are inter x hidden, down hidden x inter       */
  int64_t seqs;     /* calibration sequences, >= 1                                                */
  int64_t seq_len;  /* tokens per sequence, >= 1; attention is causal within each sequence        */
  double eps;       /* RMSNorm epsilon, >= 0: y = x / sqrt(mean(x^2) + eps) over each token's row  */
} gptq_block_shape_t;

/* One layer of the block: its weights in, its gptq_quantize_layer outputs out. */
typedef struct {
  const void *W;    /* device [rows x d] of w_dtype, row-major with ld = d; not modified          */
  uint8_t *codes;   /* device uint8[rows x d], original column order                              */
  float *scales;    /* device float[rows x ngroups]                                               */
  int32_t *zeros;   /* device int32[rows x ngroups]                                               */
  int32_t *g_idx;   /* device int32[d]                                                            */
  int32_t *perm;    /* device int32[d]: the processing order used (shared within a stage)         */
  double *loss;     /* device double[1]                                                           */
  int32_t w_dtype;  /* GPTQ_F32, GPTQ_F16 or GPTQ_BF16                                            */
} gptq_block_layer_t;

/* Workspace bytes for gptq_quantize_block (p->block_size is read); 0 for invalid arguments. */
size_t gptq_block_workspace_bytes(const gptq_block_shape_t *shape, const gptq_params_t *p);

/*
 * Quantizes the seven linear layers of one decoder block in the true-sequential order (GPTQ tools
 * page, "How it works", Step 9; the Technical Guide's "true_sequential" setting):
 *   stage 0: q, k, v from the Hessian of the attention input RMSNorm(X);
 *   stage 1: o from the Hessian of the attention output, recomputed through the quantized q, k, v;
 *   stage 2: gate, up from the MLP input RMSNorm(X + attn o^T), through the quantized o;
 *   stage 3: down from silu(x gate^T) * (x up^T), through the quantized gate and up.
 * Each stage forms H = 2 A^T A over all tokens, factors it once (gptq_factor) and runs
 * gptq_quantize_layer for each of its layers with that factor and order. With true_sequential = 0
 * every stage input comes from the block with its original weights (the layers are solved from
 * one unquantized forward pass). Activations are fp32. The projections and each stage's H run on
 * the fp16 matrix cores from operands split into two fp16 halves (hi + lo equals an fp32 value to
 * within 2^-22 relative; weights are scaled by a power of two first), which matches fp32 products
 * to within about their inputs' rounding. Stage inputs must stay below 65504 in magnitude (beyond
 * it H is not finite and the stage's factor fails).
 *
 *   shape   the block and calibration sizes (n = seqs * seq_len tokens).
 *   X       device [n x hidden] of x_dtype, token-major, sequence after sequence. Not modified.
 *   p       the quantization settings of every layer (as gptq_quantize_layer).
 *   layers  host array of 7 descriptors, in the order q, k, v, o, gate, up, down.
 *   Y       device float[n x hidden]: the block output through the quantized weights (the input
 *           of the next block).
 *   hess    NULL, or a host array of 4 pointers (each NULL or device float[d x d] for that stage's
 *           input width d): receives each stage's H (upper triangle authoritative).
 *   work    device workspace of gptq_block_workspace_bytes(shape, p) bytes.
 *   info    host int64[2]: on GPTQ_ENOTPD the failed stage (0..3) and pivot; otherwise {-1, 0}.
 *   stream  HIP stream; the call synchronizes it once per stage (to read each factor's status) and
 *           once per projection (to read the weight's scale): 11 times with true_sequential, 18
 *           without.
 * Returns GPTQ_EINVAL for bad shapes, pointers or settings, GPTQ_ENOMEM for a short workspace,
 * GPTQ_ENOTPD (see info) when a stage's damped Hessian is not positive definite, and the statuses
 * of the calls it makes. Outputs of later stages are undefined after an error.
 */
gptq_status_t gptq_quantize_block(const gptq_block_shape_t *shape, const void *X, int32_t x_dtype,
                                  const gptq_params_t *p, int32_t true_sequential, const gptq_block_layer_t *layers,
                                  float *Y, float *const *hess, void *work, size_t work_bytes, int64_t *info,
                                  void *stream);

/*
 * Workspace bytes for a call: kind GPTQ_WS_HESSIAN (a = n_tok of the chunk), GPTQ_WS_FACTOR (a unused)
 * or GPTQ_WS_QUANTIZE (a = rows; p->block_size is read). Returns 0 for invalid arguments.
 */
size_t gptq_workspace_bytes(int32_t kind, int64_t a, int64_t d, const gptq_params_t *p);

/* A static, human-readable name for a status code. */
const char *gptq_status_string(gptq_status_t s);

#ifdef __cplusplus
}
#endif

#endif /* GPTQ_H */
