/*
 * qgalore.h — C ABI of the MI355X (gfx950) Q-GaLore optimizer-step library.
 *
 * The method (AIMech curated page "Q-GaLore (Quantized GaLore with INT4 Projection and
 * Layer-Adaptive Low-Rank Gradients)"; paper Section 3.2 for the update rule, Section 3.1 /
 * Equation (5) for the subspace test): for each linear layer with weight W (m x n) and
 * gradient G (m x n), a rank-r projection P (m x r) stored in INT4 projects the gradient,
 * R = P^T G; Adam runs on R with first and second moments M, V (r x n) stored in INT8; the
 * Adam update N is back-projected, U = alpha * P N, and added into the INT8 weights with
 * unbiased stochastic rounding. A layer's projection is refreshed from an SVD at an
 * interval that doubles whenever the subspace similarity
 *     CosSim(P_t, P_prev) = (1/r) * sum_i sigma_i(P_t^T P_prev)
 * exceeds gamma (default 0.4).
 *
 * Number formats (fixed by this library; the pages leave them open):
 *   G        bf16, m x n row-major (bit patterns as uint16).
 *   W_q      int8, m x n row-major, codes in [-127, 127].
 *   W_scale  fp32, one scale per group of 256 consecutive flat elements of W
 *            (ceil(m*n/256) entries). Read-only during a step.
 *   P_q      INT4, m x r row-major, two codes per byte (flat element 2k in the low nibble
 *            of byte k, 2k+1 in the high nibble, two's complement, codes in [-7, 7]);
 *            ceil(m*r/2) bytes.
 *   P_scale  fp32, ceil(m*r/256) group scales of P, finite and of magnitude below 2^125
 *            (the INT4 dequantization computes q*s as one fma with -8*s).
 *            Two other projection formats can be selected per layer (qg_p_format): INT8
 *            codes in [-127, 127] (m*r bytes) with the same group scales, or bf16 values
 *            (m*r uint16, P_scale unused).
 *   M_q, V_q int8, r x n row-major; M_scale, V_scale fp32, ceil(r*n/256) group scales.
 *            All four are rewritten in place by every step (absmax requantization).
 * Group quantization everywhere is symmetric absmax over 256 flat elements:
 *   s = absmax/qmax, q = clamp(round_half_even(x * (1/s)), -qmax, qmax), s = 0 -> q = 0.
 *
 * Arithmetic of one step (every fp32 operation rounded to nearest-even, no contraction):
 *   P~  = bf16(q_P * s_P)                      (dequantized projection, bf16 operand)
 *   R   = P~^T G                               (fp32 accumulation on bf16 MFMA)
 *   m1  = b1*(q_M*s_M) + (1-b1)*R ;  v1 = b2*(q_V*s_V) + (1-b2)*(R*R)
 *   N   = -(lr * (m1/(1-b1^t))) / (sqrt(v1/(1-b2^t)) + eps) ;  N~ = bf16(N)
 *   M, V <- absmax INT8 requantization of m1, v1 (the update uses the fresh fp32 values)
 *   U   = alpha * (P~ N~)                      (fp32 accumulation on bf16 MFMA)
 *   d   = (W_q + U * (1/s_W)) + u ;  W_q <- clamp(floor(d), -127, 127)  (d finite;
 *         otherwise W_q is left unchanged)
 *   u   = 16-bit uniform in [0,1) from Philox4x32-10 (Salmon et al., SC'11):
 *         key = (seed & 0xffffffff, seed >> 32), counter = (j >> 3, i, t, layer_id),
 *         word (j >> 1) & 3, low half for even j and high half for odd j, times 2^-16.
 *
 * Conventions for every entry point below:
 *   - Tensor pointers are DEVICE pointers owned by the caller; the library keeps no tensor
 *     state. Inputs are read-only unless stated. No two pointers may alias.
 *   - `stream` is a hipStream_t (NULL = the null stream). Step entry points are
 *     asynchronous on that stream.
 *   - Errors are returned as qg_status; nothing is thrown or aborted across the ABI.
 *     Arguments are validated before any HIP call. HIP failures return QG_ERR_HIP and
 *     qgalore_last_error() (thread-local) holds the text.
 *   - Base pointers of G, W_q, M_q, V_q, R_out, U_out and workspaces must be 16-byte
 *     aligned; scale arrays and P_q 4-byte aligned (QG_ERR_ALIGN otherwise).
 */
#ifndef QGALORE_H
#define QGALORE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QG_OK = 0,
  QG_ERR_NULL = 1,       /* a required pointer is NULL */
  QG_ERR_SHAPE = 2,      /* m, n, r out of range: need 1 <= r <= m, r % 8 == 0, and
                            m*n, r*n, m*r <= 2^29 (every per-layer tensor below 2 GiB) */
  QG_ERR_ALIGN = 3,      /* a base pointer breaks the alignment rule above */
  QG_ERR_WORKSPACE = 4,  /* workspace smaller than the size query returns */
  QG_ERR_ARG = 5,        /* step out of [1, 2^32), non-finite or out-of-range hyperparameter */
  QG_ERR_HIP = 6,        /* a HIP runtime call or kernel launch failed */
  QG_ERR_NO_DEVICE = 7   /* no HIP device is present */
} qg_status;

/* Storage format of a projection P. INT4 is the method's (AIMech Q-GaLore page, mechanism
 * claim "INT4 projection and INT8 stochastic rounding", paper Section 3.2: a quarter of the
 * bf16 projection's memory); the other two are the projections it is compared with on the
 * same page (identity notes): GaLore's 16-bit projection and the 8-bit one of the Q-GaLore
 * baseline. */
typedef enum {
  QG_P_INT4 = 0,   /* P_q: ceil(m*r/2) bytes of packed INT4 codes; P_scale: group scales */
  QG_P_INT8 = 1,   /* P_q: m*r int8 codes in [-127, 127]; P_scale: group scales */
  QG_P_BF16 = 2    /* P_q: m*r bf16 values (16-byte aligned); P_scale: unused (may be NULL) */
} qg_p_format;

/* Where an INT4 projection is dequantized (the step's first stage, P~ = bf16(q_P * s_P)).
 * INLINE: inside the two MFMA kernels, on the way into LDS (the packed codes and their scales
 * reach LDS by DMA and are converted there): no bf16 copy of P exists outside LDS and the
 * workspace holds none (m*r*2 bytes less per layer). It needs a rank r with r % 32 == 0 and
 * (r % 128 == 0 or 256 % r == 0); other ranks, and INT8 projections, fall back to PASS.
 * PASS: a separate kernel writes the bf16 P~ to the workspace at the start of the step and
 * both MFMA kernels read it. AUTO is PASS, the faster one on MI355X (about 10% of the step at
 * rank 1024, 4% at rank 128, on the LLaMA-7B layer set); INLINE trades that for memory. The
 * results are bit-identical either way. */
typedef enum {
  QG_DEQUANT_AUTO = 0,
  QG_DEQUANT_INLINE = 1,
  QG_DEQUANT_PASS = 2
} qg_dequant_mode;

/* Per-layer description for qgalore_step. */
typedef struct {
  int64_t m, n, r;          /* W, G: m x n; P: m x r; M, V: r x n */
  uint32_t layer_id;        /* Philox counter word 3: unique per layer within a model */
  float lr, beta1, beta2, eps, alpha;   /* Adam (0 <= beta < 1, eps >= 0) and the update scale */
  float *M_scale, *V_scale; /* fp32[ceil(r*n/256)], read and rewritten in place */
  float *R_out;             /* optional fp32 r x n: the projected gradient R (NULL = skip) */
  float *U_out;             /* optional fp32 m x n: the back-projected update U (NULL = skip).
                             * With U skipped and alpha a power of two in [2^-125, 1], the
                             * rounding takes U / s_W as S * fl(alpha / s_W) (S = P~ N~): the
                             * same number wherever alpha S is normal or zero, so the W codes
                             * match those of a call that writes U (which rounds fl(alpha S)). */
  void *workspace;          /* caller-owned device scratch, >= qgalore_workspace_bytes() */
  size_t workspace_bytes;
  void *stream;             /* hipStream_t */
  int32_t p_format;         /* qg_p_format of P_q / P_scale (0 = INT4) */
  int32_t dequant_mode;     /* qg_dequant_mode (0 = AUTO); QG_ERR_ARG outside the enum */
} qg_layer_desc;

/* Device scratch one qgalore_step call needs for an m x n layer of rank r, for any format and
 * dequant mode (the largest case: a bf16 copy of P in the workspace). 0 for an invalid shape. */
size_t qgalore_workspace_bytes(int64_t m, int64_t n, int64_t r);
/* The same for the layer as `desc` describes it (m, n, r, p_format, dequant_mode): without the
 * bf16 copy of P when the projection is dequantized inline or stored in bf16. 0 when invalid. */
size_t qgalore_layer_workspace_bytes(const qg_layer_desc *desc);

/* One Q-GaLore optimizer step for one layer (AIMech Q-GaLore page, mechanism claim "INT4
 * projection and INT8 stochastic rounding", paper Section 3.2). Updates W_q, M_q, V_q and
 * the desc's M_scale, V_scale in place; `step` is the 1-based Adam step t (1 <= t < 2^32);
 * `seed` keys the stochastic rounding. Asynchronous on desc->stream. Concurrent calls on
 * one device must use distinct workspaces. */
qg_status qgalore_step(const qg_layer_desc *desc, const uint16_t *G, int8_t *W_q,
                       const float *W_scale, const uint8_t *P_q, const float *P_scale,
                       int8_t *M_q, int8_t *V_q, int64_t step, uint64_t seed);

/* For callers that cannot allocate device memory (code under graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): qgalore_step with the scratch taken from a fixed
 * device array inside the library instead of desc->workspace (ignored, as is
 * desc->workspace_bytes). The array holds QG_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU, stays
 * resident until the process ends, and is shared by every call on that GPU: calls that overlap
 * on one GPU race and must be serialized by the caller. A layer whose workspace
 * (qgalore_layer_workspace_bytes) exceeds the array returns QG_ERR_WORKSPACE, with the sizes
 * in qgalore_last_error(); every 7B-shaped layer up to rank 1024 fits. Allocates nothing;
 * otherwise as qgalore_step (same validation, results identical to it). */
#define QG_NOALLOC_SCRATCH_BYTES (64u << 20)
qg_status qgalore_step_noalloc(const qg_layer_desc *desc, const uint16_t *G, int8_t *W_q,
                               const float *W_scale, const uint8_t *P_q, const float *P_scale,
                               int8_t *M_q, int8_t *V_q, int64_t step, uint64_t seed);

/* ------------------------------------------------------------------------------------
 * Grouped step: one launch per kernel over a whole set of layers (the per-layer step of
 * the same page, applied to every linear layer of a model at once).
 * ---------------------------------------------------------------------------------- */
typedef struct {
  qg_layer_desc desc;       /* workspace / workspace_bytes / stream are ignored here */
  const uint16_t *G;
  int8_t *W_q;
  const float *W_scale;
  const uint8_t *P_q;
  const float *P_scale;
  int8_t *M_q;
  int8_t *V_q;
} qg_layer;

typedef struct qg_plan qg_plan;

/* Validates every layer and uploads a layer table to the current device (the only
 * allocation: a small table, freed by qgalore_plan_destroy). All layers must share beta1
 * and beta2. The tensors named by `layers` must stay valid while the plan is used. */
qg_status qgalore_plan_create(const qg_layer *layers, int32_t count, qg_plan **out);
/* Device scratch a qgalore_plan_step call needs. */
size_t qgalore_plan_workspace_bytes(const qg_plan *plan);
/* One optimizer step over every layer of the plan, asynchronous on `stream`. The workspace
 * carries nothing from one call to the next (unless qgalore_plan_cache_proj is on), so plans
 * stepped one after another on one stream may share one workspace of the largest size: a
 * large layer set can step as several plans over windows of its layers, holding the
 * step-transient update N~ and dequantized P~ of one window at a time. */
qg_status qgalore_plan_step(qg_plan *plan, int64_t step, uint64_t seed, void *workspace,
                            size_t workspace_bytes, void *stream);
qg_status qgalore_plan_destroy(qg_plan *plan);

/* Per-kernel timing of a plan (benchmark instrumentation). After
 * qgalore_plan_enable_timing(plan, max_steps) each qgalore_plan_step records hipEvents around
 * each of its four launches, for up to max_steps steps; the events are created here and owned
 * by the plan (max_steps = 0 frees them and disables timing). qgalore_plan_kernel_times waits
 * for the recorded events, writes each kernel's mean duration over the recorded steps to
 * out_ms[0..3] (milliseconds, in launch order: INT4 dequant of P, projection, Adam,
 * back-projection with the rounding) and the number of steps to *steps, then clears the
 * record. */
qg_status qgalore_plan_enable_timing(qg_plan *plan, int32_t max_steps);
qg_status qgalore_plan_kernel_times(qg_plan *plan, float out_ms[4], int32_t *steps);

/* Keeping dequantized projections between steps. A step dequantizes every INT4 (or INT8)
 * projection into its bf16 copy in the workspace; a projection changes only when the
 * schedule refreshes it, so with caching on (enable = 1) a step dequantizes only the layers
 * marked by qgalore_plan_proj_changed since the previous step (plus all of them on the
 * first step, and whenever the workspace pointer differs from the previous step's).
 * Caller's contract while caching is on: call qgalore_plan_proj_changed(plan, layer) after
 * writing a layer's P_q or P_scale and before the next step, and let nothing but the plan's
 * steps write the workspace. Off (the default), every step dequantizes every projection.
 * `layer` indexes the qg_layer array given to qgalore_plan_create (QG_ERR_ARG outside it). */
qg_status qgalore_plan_cache_proj(qg_plan *plan, int32_t enable);
qg_status qgalore_plan_proj_changed(qg_plan *plan, int32_t layer);

/* ------------------------------------------------------------------------------------
 * Subspace similarity (AIMech Q-GaLore page, mechanism claim "layer-adaptive subspace
 * cosine schedule", paper Section 3.1, Equation (5)).
 * ---------------------------------------------------------------------------------- */
typedef struct {
  int64_t m, r;             /* P is m x r */
  const uint8_t *q;         /* codes (or bf16 values), layout as P_q above */
  const float *scale;       /* ceil(m*r/256) group scales (unused for bf16) */
  int32_t format;           /* qg_p_format; both projections of a pair share it */
} qg_proj;

size_t qgalore_cossim_workspace_bytes(int64_t m, int64_t r);
/* CosSim of two stored projections (each dequantized and rounded to bf16 as the step uses
 * it): C = P~_new^T P~_old, then (1/r) * nuclear norm of C as trace(X^T C) with X the polar
 * factor of C from a Newton-Schulz iteration (bf16 MFMA products for the iterations that
 * lift small singular values, then hi/lo split products for fp32-level orthogonality);
 * absolute error about 1e-5. Writes one fp32 to `out_dev` (device), asynchronously. */
qg_status qgalore_cossim_async(const qg_proj *P_new, const qg_proj *P_old, void *workspace,
                               size_t workspace_bytes, void *stream, float *out_dev);
/* Many pairs at once (the layers whose refresh falls due at the same step): all pairs must
 * share the rank r (their row counts may differ); out_dev[k] receives CosSim(P_new[k],
 * P_old[k]). The workspace holds up to 32 pairs at a time; larger batches run in chunks. */
size_t qgalore_cossim_batch_workspace_bytes(int64_t r, int32_t count);
qg_status qgalore_cossim_batch(const qg_proj *P_new, const qg_proj *P_old, int32_t count,
                               void *workspace, size_t workspace_bytes, void *stream,
                               float *out_dev);
/* One pair, then synchronizes `stream` and stores the value in *out_host. */
qg_status qgalore_cossim(const qg_proj *P_new, const qg_proj *P_old, void *workspace,
                         size_t workspace_bytes, void *stream, float *out_host);

/* INT4 group quantization of an fp32 m x r projection (the format of P_q/P_scale above;
 * used when a refresh installs a new projection). Asynchronous on `stream`. */
qg_status qgalore_quantize_proj(const float *P, int64_t m, int64_t r, uint8_t *P_q,
                                float *P_scale, void *stream);
/* The same with INT8 codes (QG_P_INT8: m*r bytes of codes in [-127, 127]). */
qg_status qgalore_quantize_proj_int8(const float *P, int64_t m, int64_t r, int8_t *P_q,
                                     float *P_scale, void *stream);

/* ------------------------------------------------------------------------------------
 * Subspace refresh on the GPU (AIMech curated page on Q-GaLore, definition paragraph and
 * mechanism claims: a layer's projection holds the rank-r leading singular vectors of its
 * gradient, recomputed by an SVD at each refresh and stored in INT4).
 *
 * P (m x r) = the r leading left singular vectors of G (bf16 m x n), approximated by a
 * randomized range finder with power iterations (Halko, Martinsson and Tropp, SIAM Review
 * 2011, Algorithms 4.4 and 5.1):
 *   Y = G Omega, Q = orth(Y); power_iters times: Z = orth(G^T Q), Q = orth(G Z);
 *   B = Q^T G; B B^T = V diag(sigma^2) V^T; P = Q V[:, :r],
 * with orth() a CholeskyQR2 in fp32, the products with G on bf16 MFMA (fp32 bases entered
 * as bf16 hi + lo parts), and the eigenproblem of B B^T by parallel block Jacobi across
 * workgroups (blocks of 32 indices, 64 x 64 subproblems, C, V and the rotations held in
 * fp64). Sketches up to k = 136 orthonormalize with the k x k work in one workgroup per
 * step; wider ones (up to 2048) by block Gram-Schmidt with reorthogonalization (blocks of
 * 128 columns, each by CholeskyQR2, the k x k products on fp32 MFMA). Each column of
 * P is negated if needed so that its entry of largest magnitude (the first such row) is
 * positive. P is then quantized to INT4 (P_q, P_scale, as qgalore_quantize_proj).
 *   G          bf16 m x n row-major, 16-byte aligned; when n is not a multiple of 8 the
 *              library works on a zero-padded copy in the workspace.
 *   Omega      bf16 n x k row-major sketch (k = r + oversample), drawn by the caller
 *              (standard Gaussian entries); device pointer, 16-byte aligned.
 *   oversample multiple of 8, k <= 2048, k <= min(m, n); power_iters 0..8.
 *   P_out      optional fp32 m x r (16-byte aligned): P before quantization.
 *   sigma_out  optional fp32 r: the approximated leading singular values of G.
 * The result approximates the SVD's: its error grows with sigma_{k+1}/sigma_r of G and
 * shrinks with power_iters. Asynchronous on `stream` (the block Jacobi solver issues a fixed
 * number of sweeps whose kernels return at once after convergence, so nothing is read back);
 * allocates nothing. */
size_t qgalore_refresh_workspace_bytes(int64_t m, int64_t n, int64_t r, int32_t oversample);
qg_status qgalore_refresh_proj(const uint16_t *G, int64_t m, int64_t n, int64_t r,
                               const uint16_t *Omega, int32_t oversample, int32_t power_iters,
                               uint8_t *P_q, float *P_scale, float *P_out, float *sigma_out,
                               void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------------------
 * Products of a linear layer whose weight is the INT8 W_q / W_scale above (AIMech curated
 * page on Q-GaLore, limitation claim "simulated weight quantization throughput": the
 * activations stay 16-bit and the INT8 weight is dequantized inside the forward and
 * backward passes). W~ = bf16(q_W * s_W) is formed inside the kernels and never stored.
 *   X, dX   bf16 T x n row-major (T tokens, n inputs)
 *   Y, dY   bf16 T x m row-major (m outputs)
 *   G       bf16 m x n row-major (the weight gradient qgalore_step takes)
 * Each product accumulates in fp32 (bf16 MFMA) and rounds to bf16. m and n must be
 * multiples of 8; T*m, T*n and m*n at most 2^29. bf16 tensors and W_q 16-byte aligned.
 * Asynchronous on `stream`; no workspace. */
qg_status qgalore_int8_linear_fwd(const uint16_t *X, const int8_t *W_q, const float *W_scale,
                                  int64_t T, int64_t m, int64_t n, uint16_t *Y, void *stream);
qg_status qgalore_int8_linear_bwd_data(const uint16_t *dY, const int8_t *W_q,
                                       const float *W_scale, int64_t T, int64_t m, int64_t n,
                                       uint16_t *dX, void *stream);
qg_status qgalore_linear_bwd_weight(const uint16_t *dY, const uint16_t *X, int64_t T, int64_t m,
                                    int64_t n, uint16_t *G, void *stream);

/* ------------------------------------------------------------------------------------
 * Per-layer refresh schedule (host only; same page and claim as CosSim). A refresh falls
 * due when t >= next_refresh. At each refresh after the first, a similarity above gamma
 * doubles the interval; the next refresh is then t + interval.
 * ---------------------------------------------------------------------------------- */
typedef struct {
  int64_t delta;            /* current refresh interval */
  int64_t next_refresh;     /* step of the next refresh */
  int64_t count;            /* refreshes (SVDs) done so far */
  float gamma;              /* similarity threshold */
  float last_cossim;        /* similarity seen at the last refresh (NaN before the second) */
} qg_sched;

qg_status qgalore_sched_init(qg_sched *s, int64_t delta0, float gamma);
/* 1 when a refresh is due at step t, else 0 (-1 for a NULL schedule). */
int32_t qgalore_sched_due(const qg_sched *s, int64_t t);
/* Records a refresh at step t with similarity `cossim` (ignored at the first refresh).
 * *doubled (optional) is set to 1 when the interval doubled. */
qg_status qgalore_sched_refresh(qg_sched *s, int64_t t, float cossim, int32_t *doubled);

/* ------------------------------------------------------------------------------------
 * Calibration of the compute roofline (not part of a step): the bf16 MFMA rate the chip
 * sustains on given operand data, since the clock under sustained matrix load depends on
 * the operands' switching activity. `grid` workgroups of 4 waves; every wave reads 4 A and
 * 4 B MFMA fragments (8 bf16 each, consecutive 16-byte chunks of `operands`, wrapping
 * around) once and runs `iters` rounds of 16 v_mfma_f32_32x32x16_bf16 (32768 flops each),
 * so a launch does grid * 4 * iters * 16 * 32768 flops. out: grid * 256 floats (one
 * checksum per lane). operands: n_elems bf16, n_elems a multiple of 8 (>= 8), 16-byte
 * aligned. grid in [1, 65536], iters in [1, 2^20]. Asynchronous on `stream`.
 * ---------------------------------------------------------------------------------- */
qg_status qgalore_mfma_probe(const uint16_t *operands, int64_t n_elems, float *out, int32_t grid,
                             int32_t iters, void *stream);

/* ------------------------------------------------------------------------------------ */
const char *qgalore_status_str(qg_status s);
const char *qgalore_last_error(void);   /* thread-local text of the last QG_ERR_HIP (or of
                                           qgalore_step_noalloc's QG_ERR_WORKSPACE) */
const char *qgalore_version(void);

#ifdef __cplusplus
}
#endif
#endif /* QGALORE_H */
