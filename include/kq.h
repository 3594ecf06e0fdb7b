/*
 * kq.h -- KronQ per-layer quantization on AMD Instinct MI355X (gfx950).
 *
 * A C ABI over hand-written HIP kernels. Every argument is a plain pointer or
 * a size; no framework types cross this boundary.
 *
 * Sources cited below (page title, then section):
 *   [KQ-en]   "KronQ: LLM Quantization via Kronecker-Factored Hessian",
 *             gptget.net English summary: Methodology, Technical Contribution.
 *   [KQ-zh]   gptget.net Chinese summary of the paper: 方法论 (methodology).
 *   [KQ-news] "KronQ: Kronecker Hessians break GPTQ's 2-bit wall", aimodeling.com.
 *   [KQ-art]  wmrh.cn article on KronQ, sections 二, 三, 四, 六, 七, 八 and the Q&A.
 *
 * Conventions shared by every entry point
 *   - Pointers are DEVICE pointers unless a comment says "host". The caller
 *     owns every buffer; the library allocates no device memory. Scratch space
 *     is passed in as `ws` / `ws_bytes` after a kq_workspace_size() query.
 *   - Matrices are row-major. Covariances are float32, d x d, leading
 *     dimension d, and both triangles are valid.
 *   - `stream` is a hipStream_t (NULL = the null stream). Calls enqueue work on
 *     it and return; nothing is synchronised unless stated.
 *   - Argument errors are reported synchronously, before anything is enqueued,
 *     as KQ_EINVAL / KQ_EUNSUPPORTED; kq_last_error() then holds a message.
 *     A failed launch returns KQ_EDEVICE. Numerical failure inside a kernel is
 *     reported through a device `info` word (0 = success).
 *   - Buffers passed to one call must not overlap unless stated ("in place").
 */
#ifndef KQ_H_
#define KQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KQ_OK = 0,
  KQ_EINVAL = 1,        /* bad argument (shape, pointer, flag, precondition) */
  KQ_ENOTPD = 2,        /* reported by the host-side helpers when info != 0 */
  KQ_EINFEASIBLE = 3,   /* bit budget below min(choices) for every sub-layer */
  KQ_EDEVICE = 4,       /* HIP runtime error while enqueueing */
  KQ_EUNSUPPORTED = 5   /* valid request outside what the kernels implement */
} kq_status;

/* Element types of the weight input of kq_biip_rotate. */
enum { KQ_BF16 = 0, KQ_F32 = 1, KQ_F64 = 2 };

/* kq_biip_rotate flags. */
enum {
  KQ_BIIP_INPUT = 1,    /* process the input side (columns of W) with H_X */
  KQ_BIIP_OUTPUT = 2,   /* process the output side (rows of W) with H_G */
  KQ_BIIP_SCALE = 4,    /* diagonal rescale of each processed side before its rotation */
  KQ_BIIP_INVERSE = 8   /* map a rotated weight back: W = S_G^-1 U_G^T W'' U_X S_X^-1 */
};

/* kq_sensitivity modes. */
enum { KQ_SCORE_KRONQ = 0, KQ_SCORE_HX_ONLY = 1 };

/* kq_workspace_size operations. */
enum { KQ_OP_ACCUMULATE_COV = 0, KQ_OP_BIIP = 1, KQ_OP_CHOLESKY = 2, KQ_OP_OBS = 3, KQ_OP_DECODE = 4,
       KQ_OP_LOSS = 5, KQ_OP_XCOV = 6, KQ_OP_GPTAQ = 7 };

#define KQ_MAX_ODD 63         /* largest odd factor m of a rotated dimension */
#define KQ_MAX_ROT_DIM 32768  /* largest rotated dimension n = m * 2^k */
#define KQ_DECODE_MAX_TOKENS 4  /* tokens per kq_decode_matvec call */
#define KQ_DECODE_MAX_LAYERS 4  /* layers per kq_decode_matvec_group call */
#define KQ_DECODE_NOALLOC_SCRATCH 2228224  /* bytes of the fixed scratch of kq_decode_matvec_group_noalloc */

/*
 * Rotation of one side: U = (Q_m kron H_p / sqrt(p)) diag(sigma), n = m * p,
 * p = 2^log2p, m odd. H_p is the Sylvester Hadamard matrix,
 * H_p[b][b'] = (-1)^popcount(b & b'); index i = a * p + b (a < m, b < p).
 * [KQ-art] 七 and Q&A: the incoherence rotation is a Hadamard transform of
 * O(d log d) cost; [KQ-zh] 方法论: a random orthogonal transform. The random
 * draw (sigma, Q_m) is an input, made by the caller.
 */
typedef struct {
  int64_t n;              /* dimension of this side */
  int32_t m;              /* odd factor, 1 <= m <= KQ_MAX_ODD */
  int32_t log2p;          /* n = m << log2p */
  const int8_t* signs;    /* device [n], each +1 or -1 */
  const double* q;        /* device [m * m], row-major orthogonal matrix Q_m */
} kq_rot;

/* Library version string (host, static storage). */
const char* kq_version(void);
/* Text of a status code (host, static storage). */
const char* kq_status_string(kq_status s);
/* Message of the last error raised on the calling thread (host, thread-local). */
const char* kq_last_error(void);

/*
 * Kernel timing (diagnostics, host calls). kq_timing_enable(filter) clears the
 * record and, while enabled, brackets every launch of a kernel whose name
 * contains `filter` ("" = all kernels; "a|b" = names containing a or b) with
 * HIP events on that launch's
 * stream; NULL disables. kq_timing_query(name, ...) waits for the recorded
 * events of kernels whose name contains `name` and returns the number of
 * launches and their summed duration in milliseconds. Not thread safe
 * against concurrent launches from other host threads.
 */
kq_status kq_timing_enable(const char* filter);
kq_status kq_timing_query(const char* name, int64_t* launches, double* total_ms);

/*
 * Bytes of scratch space an operation needs (0 = none).
 *   KQ_OP_ACCUMULATE_COV: d0 = rows, d1 = d
 *   KQ_OP_BIIP:           d0 = dout, d1 = din
 *   KQ_OP_CHOLESKY:       d0 = d
 *   KQ_OP_OBS:            d0 = dout, d1 = din, d2 = block
 *   KQ_OP_DECODE:         d0 = dout (kq_decode_matvec_group: the layers' total), d1 = din, d2 = tokens
 *   KQ_OP_LOSS:           d0 = dout, d1 = din
 *   KQ_OP_XCOV:           d0 = rows, d1 = d
 *   KQ_OP_GPTAQ:          d0 = dout, d1 = din
 *   (kq_biip_transform of an n x n matrix uses KQ_OP_BIIP with d0 = d1 = n)
 * Returns (size_t)-1 for invalid sizes.
 */
size_t kq_workspace_size(int32_t op, int64_t d0, int64_t d1, int64_t d2);

/*
 * kq_accumulate_cov -- H <- alpha * A^T A + beta * H   (symmetric rank-k update)
 *
 * With A = X (calibration activations) and alpha = 1/N this forms H_X, the
 * activation covariance GPTQ uses as its Hessian proxy; with A = G (gradients
 * of the layer output from one backward pass) it forms H_G. The weight
 * Hessian is approximated by H_X kron H_G ([KQ-art] 二; [KQ-news];
 * [KQ-en] Methodology). Call once per token chunk with beta = 0 and then 1.
 *
 *   a      device, bf16 bit patterns, [rows, d] with row pitch lda elements (lda >= d)
 *   rows   number of token rows, >= 0 (0: H <- beta * H)
 *   h      device float32 [d, d]; read only when beta != 0; both triangles written
 *   ws     scratch of kq_workspace_size(KQ_OP_ACCUMULATE_COV, rows, d, 0) bytes
 *          (the float32 partial sums of every 16384-row slice when they fit in
 *          64 GiB, else of one launch's slices plus a float64 running sum; the
 *          environment variable KQ_COV_KEEP_ALL_MAX_BYTES, a decimal byte count,
 *          replaces the 64 GiB when set, for kq_workspace_size and the call
 *          alike: keep it unchanged between the two)
 * bf16 products are exact; sums run in float32 within token slices of 16384
 * rows and in float64 across slices; the result is rounded once to float32.
 */
kq_status kq_accumulate_cov(const uint16_t* a, int64_t rows, int64_t d, int64_t lda, float alpha,
                            float beta, float* h, void* ws, size_t ws_bytes, void* stream);

/*
 * kq_accumulate_xcov -- C <- alpha * A^T B + beta * C_in   (cross second moment)
 *
 * Row f2, the GPTAQ base quantizer: KronQ's column update is GPTAQ's, which
 * corrects GPTQ for the drift between the inputs of the full-precision layer
 * and those of the partly quantized model ([KQ-art] 四, 八; the pages give no
 * formula). With A = Xt (full-precision inputs), B = X (quantized-model
 * inputs, the same tokens), alpha = 1/N, beta = -1 and C_in = H_X from
 * kq_accumulate_cov of X, it forms the drift moment D = (Xt - X)^T X / N.
 *   a, b   device, bf16 bit patterns, [rows, d] with row pitches lda, ldb (>= d)
 *   rows   number of token rows, >= 0 (0: C <- beta * C_in)
 *   c_in   device float32 [d, d]; read only when beta != 0 (then not NULL); may equal c
 *   c      device float32 [d, d]; every entry written
 *   ws     scratch of kq_workspace_size(KQ_OP_XCOV, rows, d, 0) bytes
 * Arithmetic as kq_accumulate_cov (exact bf16 products, float32 within token
 * slices of 16384 rows, float64 across slices), over every 256 x 256 tile of
 * the square; alpha * A^T B is rounded to float32 before beta * C_in is added
 * (and the sum rounded again), so identical inputs with C_in from
 * kq_accumulate_cov and beta = -1 give exactly zero (both sum the same float32
 * slice partials in slice order in float64, however the slices are split into
 * launches).
 */
kq_status kq_accumulate_xcov(const uint16_t* a, const uint16_t* b, int64_t rows, int64_t d, int64_t lda,
                             int64_t ldb, float alpha, float beta, const float* c_in, float* c, void* ws,
                             size_t ws_bytes, void* stream);

/*
 * kq_biip_transform -- M <- U S^-1 M S^-1 U^T   (the input-side map of BiIP)
 *
 * The map kq_biip_rotate applies to H_X, for another second moment of the same
 * inputs (row f2: the drift moment D), with the scales of that forward call.
 *   m      device float32 [n, n], in place (need not be symmetric)
 *   rot    HOST pointer to the input-side rotation spec (its n must match)
 *   s      device float64 [n]: the s_x of the forward call; NULL means 1
 *   ws     scratch of kq_workspace_size(KQ_OP_BIIP, n, n, 0) bytes
 * Precision as kq_biip_rotate (float64 on chip, float32 between passes).
 */
kq_status kq_biip_transform(float* m, int64_t n, const kq_rot* rot, const double* s, void* ws, size_t ws_bytes,
                            void* stream);

/*
 * kq_gptaq_target -- W <- W + W triu(D R^T, 1) R   (GPTAQ's drift correction)
 *
 * Row f2. Reading of GPTAQ taken ([KQ-art] 四, 八): each column q's drift
 * w_q dx_q is compensated by least squares on the later columns' inputs
 * (GPTQ's damping as ridge), which moves them by w_q D_{q,>q} H~_{>q,>q}^-1;
 * with R^T R = H~^-1 the trailing inverse is R_{>q,>q}^T R_{>q,>q}, so all of
 * them together are W P, P = triu(D R^T, 1) R. GPTQ's sweep (kq_obs_quantize
 * with the same R) then runs on the result. Without drift (D = 0) W is unchanged.
 *   w      device float64 [dout, din], in place (W'' of kq_biip_rotate)
 *   d2     device float32 [din, din]: D'' (kq_accumulate_xcov, then kq_biip_transform)
 *   r      device float32 [din, din]: R of kq_cholesky_inv on H_X'' (upper, zero below)
 *   info   device int32 (may be NULL): set to 1 when a corrected weight is
 *          not finite (a NaN or Inf in the drift moment, R or W reaches every
 *          later column); the caller sets it to 0 first. W must then not go
 *          to the sweep: its codes would be meaningless.
 *   ws     scratch of kq_workspace_size(KQ_OP_GPTAQ, dout, din, 0) bytes
 * Three float64 MFMA products with fixed summation order (deterministic).
 */
kq_status kq_gptaq_target(double* w, const float* d2, const float* r, int64_t dout, int64_t din, int32_t* info,
                          void* ws, size_t ws_bytes, void* stream);

/*
 * kq_sensitivity -- score = tr(H_G) * tr(H_X), or tr(H_X) alone
 *
 * The sub-layer sensitivity of [KQ-news] and [KQ-art] 三/六, computed on the
 * raw (pre-BiIP, undamped) covariances. KQ_SCORE_HX_ONLY gives the H_X-only
 * ranking, which ties for sub-layers sharing an input (q/k/v).
 *   h_x    device float32 [din, din]
 *   h_g    device float32 [dout, dout]; may be NULL with KQ_SCORE_HX_ONLY
 *   score  device float64 [1], written
 * Diagonals are summed in float64 in a fixed order (deterministic).
 */
kq_status kq_sensitivity(const float* h_x, int64_t din, const float* h_g, int64_t dout, int32_t mode,
                         double* score, void* stream);

/*
 * kq_allocate_bits -- mixed-precision bit widths from sensitivity scores (HOST)
 *
 * [KQ-art] 六: the most sensitive sub-layers are upgraded first at a fixed
 * average bit count. Rule: budget = floor(target_millibits * sum(n) / 1000)
 * bits, in exact 128-bit integer arithmetic (sum(n) up to 2^56); every
 * sub-layer starts at min(choices); visiting sub-layers by score (highest
 * first, ties by lower index), each is raised to the largest choice that keeps
 * sum(n_l * b_l) within the budget.
 *   score       host float64 [n_layers]
 *   n_params    host int64 [n_layers], each > 0
 *   choices     host int32 [n_choices], each in [2, 8]
 *   bits_out    host int32 [n_layers], written on KQ_OK
 * Returns KQ_EINFEASIBLE when min(choices) * sum(n) exceeds the budget and
 * KQ_EINVAL when a score is NaN or infinite (a non-finite covariance, e.g. from
 * a NaN in X, cannot rank a sub-layer). Runs entirely on the host and needs no
 * device.
 */
kq_status kq_allocate_bits(const double* score, const int64_t* n_params, int32_t n_layers,
                           const int32_t* choices, int32_t n_choices, int64_t target_millibits,
                           int32_t* bits_out);

/*
 * kq_biip_rotate -- bidirectional incoherence processing (BiIP)
 *
 * Forward (flags without KQ_BIIP_INVERSE):
 *   s_x = diag(H_X)^(1/4) (1 where the diagonal is <= 0), s_g likewise from H_G,
 *   W''   = U_G S_G W S_X U_X^T
 *   H_X'' = U_X S_X^-1 H_X S_X^-1 U_X^T      (in place)
 *   H_G'' = U_G S_G^-1 H_G S_G^-1 U_G^T      (in place)
 * The input side is processed with H_X, the output side with H_G ([KQ-art]
 * 三); the diagonal rescale precedes the rotation ([KQ-art] 八). A side
 * without its flag uses s = 1 and U = I; KQ_BIIP_SCALE off keeps the rotation
 * but sets s = 1. The map preserves tr(dW H_X dW^T H_G). H_G is not needed
 * after this call: the column sweep never reads it ([KQ-art] 四, 七).
 *
 * Inverse (KQ_BIIP_INVERSE): w_out = S_G^-1 U_G^T w U_X S_X^-1 with the s_x,
 * s_g of the forward call as inputs; h_x and h_g are not used (may be NULL).
 *
 *   w        device [dout, din] of type w_dtype (forward: any; inverse: KQ_F64)
 *   w_out    device float64 [dout, din]
 *   h_x      device float32 [din, din], in place (forward with KQ_BIIP_INPUT)
 *   h_g      device float32 [dout, dout], in place (forward with KQ_BIIP_OUTPUT)
 *   rot_in   HOST pointer to the input-side spec (n = din); used with KQ_BIIP_INPUT
 *   rot_out  HOST pointer to the output-side spec (n = dout); used with KQ_BIIP_OUTPUT
 *   s_x, s_g device float64 [din], [dout]; written (forward) or read (inverse)
 *   ws       scratch of kq_workspace_size(KQ_OP_BIIP, dout, din, 0) bytes
 * Butterflies, mixes and scales run in float64 on chip; values between the
 * passes of the transform are stored in float32 (relative error near 1e-7 in
 * W'', the precision the column sweep needs); w_out is written in float64.
 */
kq_status kq_biip_rotate(const void* w, int32_t w_dtype, int64_t dout, int64_t din, double* w_out,
                         float* h_x, float* h_g, const kq_rot* rot_in, const kq_rot* rot_out,
                         uint32_t flags, double* s_x, double* s_g, void* ws, size_t ws_bytes,
                         void* stream);

/*
 * kq_cholesky_inv -- R upper triangular with R^T R = (H + damp * mean(diag H) * I)^-1
 *
 * The GPTQ route to the column sweep: damping of 1% of the mean diagonal,
 * then the upper Cholesky factor of the inverse of the damped H_X''. It is
 * formed without an explicit inverse: H~ = V V^T with V upper (the Cholesky
 * factor of the index-reversed matrix), then R = V^-1.
 *   h      device float32 [d, d]; in: H (full symmetric); out: R (upper
 *          triangle), the strict lower triangle set to 0
 *   damp   >= 0
 *   info   device int32 [1]: 0 on success, else j + 1 where j is the first
 *          index (in elimination order, from d-1 down to 0) whose pivot was not
 *          positive or not finite; R is then undefined
 *   ws     scratch of kq_workspace_size(KQ_OP_CHOLESKY, d, 0, 0) bytes
 * Arithmetic is float32 with float64 diagonal blocks.
 */
kq_status kq_cholesky_inv(float* h, int64_t d, float damp, int32_t* info, void* ws, size_t ws_bytes,
                          void* stream);

/*
 * kq_obs_quantize -- GPTQ-style column-wise OBS on the rotated weight
 *
 * For each column j in natural order: at the first column of a group, the
 * asymmetric b-bit min-max grid of each row is taken from the current
 * (error-fed) weights of that group (group == 0: one grid per row from the
 * input weights); the scale is stored as float32 and the grid uses that
 * value; zero = round_half_even(-xmin / s) clamped to [0, 2^b - 1]; then
 *   code = clamp(round_half_even(w / s) + zero, 0, 2^b - 1),  w^ = s (code - zero)
 *   e = (w - w^) / R_jj,  w_k -= e R[j][k] for every later column k.
 * Columns inside a block of `block` columns receive the error at once; later
 * columns receive the block's errors in one product (lazy batch). H_G does
 * not appear: it cancels from the per-column update ([KQ-art] 四), so this is
 * the GPTQ update ([KQ-en] Methodology; [KQ-zh] 方法论).
 *
 *   w        device float64 [dout, din]; in: W''; out: dequantised W^'' (in place)
 *   r        device float32 [din, din], upper triangular R from kq_cholesky_inv;
 *            16-byte aligned (KQ_EINVAL otherwise)
 *   bits     2..8
 *   group    0 (one grid per row) or a divisor of block
 *   block    32, 64 or 128, dividing din
 *   codes    device uint8 [dout, din]
 *   scales   device float32 [dout, ngroups], ngroups = group ? din / group : 1
 *   zeros    device uint8 [dout, ngroups]
 *   preround device float64 [dout, din] or NULL: w / s of each entry (the
 *            argument of the rounding), for diagnostics
 *   ws       scratch of kq_workspace_size(KQ_OP_OBS, dout, din, block) bytes
 * Arithmetic is float64 throughout (float64 MFMA for the lazy-batch product).
 */
kq_status kq_obs_quantize(double* w, const float* r, int64_t dout, int64_t din, int32_t bits,
                          int32_t group, int32_t block, uint8_t* codes, float* scales,
                          uint8_t* zeros, double* preround, void* ws, size_t ws_bytes,
                          void* stream);

/*
 * kq_kron_loss -- loss = tr(dW H_X dW^T H_G), dW = W^ - W
 *
 * The layer loss under the Kronecker-factored Hessian H_X kron H_G: the
 * quadratic form vec(dW)^T (H_X kron H_G) vec(dW) with the column-major vec
 * ([KQ-en] Abstract; [KQ-news]). For validation of a quantized layer (in the
 * original frame with the raw covariances, or in the rotated frame with W'',
 * H_X'' and H_G'': BiIP preserves it).
 *   w_hat    device float64 [dout, din]
 *   w        device [dout, din] of type w_dtype (KQ_BF16, KQ_F32 or KQ_F64)
 *   h_x      device float32 [din, din], h_g device float32 [dout, dout] (full symmetric)
 *   loss     device float64 [1], written
 *   ws       scratch of kq_workspace_size(KQ_OP_LOSS, dout, din, 0) bytes
 * Float64 arithmetic (float64 MFMA) on the stored values; every sum runs in a
 * fixed order, so the result is the same on every run.
 */
kq_status kq_kron_loss(const double* w_hat, const void* w, int32_t w_dtype, int64_t dout, int64_t din,
                       const float* h_x, const float* h_g, double* loss, void* ws, size_t ws_bytes,
                       void* stream);

/*
 * kq_pack_codes -- codes of a quantized weight into 32-bit words
 *
 * The deployment path of [KQ-news] ships the quantized weight as packed int4 /
 * int2 codes. Container width c = 2 for 2-bit codes, 4 for 3- and 4-bit codes,
 * 8 for 5..8 bits; code j of a row goes to word j / (32 / c) of that row at
 * bit offset c (j mod 32 / c).
 *   codes   device uint8 [rows, cols], each < 2^bits (higher bits are not masked)
 *   packed  device uint32 [rows, cols * c / 32], written
 * cols must be a multiple of 32 / c (KQ_EINVAL otherwise).
 */
kq_status kq_pack_codes(const uint8_t* codes, int64_t rows, int64_t cols, int32_t bits,
                        uint32_t* packed, void* stream);

/*
 * kq_decode_matvec -- y = W^ x with the quantized layer in original coordinates
 *
 * W^ = S_G^-1 U_G^T W^'' U_X S_X^-1 with W^''[i][j] = scale[i][g] (code_ij - zero[i][g]),
 * g = j / group: the fused dequantization + BiIP matvec of the deployment
 * path ([KQ-news]); at inference each layer applies the two Hadamard
 * transforms, O(d log d) each ([KQ-art] Q&A). The input side (when rot_in or
 * s_x is given) runs either inside every workgroup of the matvec launch, in LDS
 * while its first rows of packed codes are in flight (no odd factor, at most one
 * workgroup per CU), or as a one-workgroup launch before it; the matvec
 * dequantizes rows as they stream in; a one-workgroup launch after it applies
 * the output side (when rot_out is given; s_g alone is applied by the matvec).
 *   packed   device uint32 [dout, din * c / 32] from kq_pack_codes
 *   scales   device float32 [dout, din / group] (group 0: [dout, 1]), as kq_obs_quantize wrote them
 *   zeros    device uint8, same shape
 *   bits     2..8; group 0 or a multiple of 16 dividing din; din a multiple of 16
 *   s_x, s_g device float64 [din], [dout] diagonal scales; NULL means 1
 *   rot_in, rot_out  HOST pointers to the rotation specs; NULL means U = I on that side
 *   x        device float32 [tokens, din], y device float32 [tokens, dout] (written)
 *   tokens   1..KQ_DECODE_MAX_TOKENS; din * tokens <= 16384 and, with rot_out,
 *            dout * tokens <= 36864 (the output side holds its tokens and the odd
 *            factor in 160 KB of LDS); KQ_EUNSUPPORTED otherwise
 *   ws       kq_workspace_size(KQ_OP_DECODE, dout, din, tokens) bytes (the matvec
 *            result before the output side, x with the input side applied when
 *            that runs as its own launch); calls sharing it must not overlap
 * Arithmetic is float32 (scales and rotation factors read as stored).
 */
kq_status kq_decode_matvec(const uint32_t* packed, const float* scales, const uint8_t* zeros,
                           int64_t dout, int64_t din, int32_t bits, int32_t group,
                           const double* s_x, const double* s_g, const kq_rot* rot_in,
                           const kq_rot* rot_out, const float* x, int64_t tokens, float* y,
                           void* ws, size_t ws_bytes, void* stream);

/* One layer of kq_decode_matvec_group: the per-layer arguments of kq_decode_matvec. */
typedef struct {
  const uint32_t* packed;  /* device uint32 [dout, din * c / 32] */
  const float* scales;     /* device float32 [dout, din / group] */
  const uint8_t* zeros;    /* device uint8, same shape */
  int64_t dout;
  const double* s_g;       /* device float64 [dout] or NULL */
  const kq_rot* rot_out;   /* HOST pointer or NULL */
  float* y;                /* device float32 [tokens, dout], written */
} kq_decode_layer;

/*
 * kq_decode_matvec_group -- kq_decode_matvec for up to KQ_DECODE_MAX_LAYERS
 * layers that read the same input x with the same input side (a transformer
 * block's q, k and v, or gate and up: the input side is keyed by the input,
 * [KQ-art] 三). The input side is applied once, one matvec launch covers every
 * layer's rows, and one launch applies the output sides, a workgroup per layer
 * that has one. Each layer's result equals what kq_decode_matvec returns for it.
 *   layers   HOST array of n_layers (1..KQ_DECODE_MAX_LAYERS) layer descriptions;
 *            each is checked as kq_decode_matvec checks its arguments
 *   din, bits, group, s_x, rot_in, x, tokens  shared, as in kq_decode_matvec
 *   ws       kq_workspace_size(KQ_OP_DECODE, sum of the layers' dout, din, tokens)
 *            bytes; calls sharing it must not overlap
 */
kq_status kq_decode_matvec_group(const kq_decode_layer* layers, int32_t n_layers, int64_t din,
                                 int32_t bits, int32_t group, const double* s_x,
                                 const kq_rot* rot_in, const float* x, int64_t tokens,
                                 void* ws, size_t ws_bytes, void* stream);

/*
 * kq_decode_matvec_group_noalloc -- kq_decode_matvec_group without a workspace argument
 *
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. Same
 * arguments, checks and result as kq_decode_matvec_group, except that the
 * scratch space lives in a fixed device array inside the library
 * (KQ_DECODE_NOALLOC_SCRATCH bytes, 2.125 MiB, one copy per GPU the library
 * runs on, held until the process ends). It covers the workspace of every call
 * that kq_decode_matvec_group accepts; a larger need returns KQ_EUNSUPPORTED.
 * The call allocates nothing: its first call on a device resolves the array's
 * device address (hipGetSymbolAddress) and keeps it.
 * Every call on one GPU shares that GPU's array, and the array keeps the last
 * call's contents (no entry needs to start at zero: every scratch value is
 * written before it is read within a call). Calls that overlap on one GPU
 * (concurrent streams, or host threads) race on it; calls on one stream are
 * ordered and safe.
 */
kq_status kq_decode_matvec_group_noalloc(const kq_decode_layer* layers, int32_t n_layers, int64_t din,
                                         int32_t bits, int32_t group, const double* s_x,
                                         const kq_rot* rot_in, const float* x, int64_t tokens,
                                         void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KQ_H_ */
