/*
 * kdn.h -- C ABI of the MI355X (gfx950) delta-rule / Kalman-Delta scan library.
 *
 * The library computes the recurrent associative-memory write of delta-rule
 * linear attention and the uncertainty-aware (Kalman) writes derived from it,
 * plus the HOLA write-magnitude score and its exact top-w key/value cache:
 *
 *   state S (d_k x d_v, float32), prediction S^T k, read-out o_t = S_t^T q_t.
 *
 *   delta write, gated residual  ("A Hippocampus for Linear Attention",
 *   sec. 3.3 eq. (5) and sec. 3.5):
 *       e_t = v_t - alpha_t S_{t-1}^T k_t,   S_t = alpha_t S_{t-1} + beta_t k_t e_t^T
 *   delta write, plain residual: e_t = v_t - S_{t-1}^T k_t, same update.
 *   Kalman write ("Kalman Delta Networks: Uncertainty-aware Associative
 *   Memory", abstract; "Memory by Design: Probabilistic Sequence Layers",
 *   abstract): the delta write with beta_t k_t replaced by the Kalman gain
 *   g_t = P-_t k_t / (k_t^T P-_t k_t + r_t), where P-_t = alpha_t^2 P_{t-1} + Q_t I,
 *   Q_t = (1 - alpha_t^2) sigma^2, and P_t = P-_t - P-_t k_t k_t^T P-_t / s_t.
 *   FULL keeps the whole d_k x d_k covariance (the recursive-least-squares
 *   update of "DeltaNet-PC", eq. (7), when alpha = 1, r = 1, sigma^2 = 0);
 *   DIAG keeps a diagonal covariance, projected after every token by
 *   mean-field inference: 1/p_i = 1/p-_i + k_i^2 / r_t. ISO keeps one variance
 *   p per head (the covariance is p I), projected onto multiples of the
 *   identity: 1/p = 1/p- + ||k_t||^2 / (d_k r_t); its gain is beta_t k_t with
 *   beta_t = p- / (p- ||k_t||^2 + r_t).
 *   score ("A Hippocampus for Linear Attention", sec. 3.3 eq. (6)):
 *       m_t = ||write_t||_F = beta_t ||e_t|| (delta), ||g_t|| ||e_t|| (Kalman).
 *
 * Conventions for every entry point
 *  - Every array argument is a DEVICE pointer owned by the caller; the library
 *    keeps no pointer after the call returns. Layouts are row-major and
 *    contiguous: sequences [B, H, L, d], per-token scalars [B, H, L], state
 *    [B, H, d_k, d_v] (S[i][j] at i*d_v + j), covariance [B, H, d_k] (DIAG),
 *    [B, H, d_k, d_k] (FULL) or [B, H] (ISO).
 *  - `stream` is a hipStream_t (NULL = the legacy default stream). Work is only
 *    enqueued; the call never synchronises. The library never allocates device
 *    memory: scratch space comes from the caller's `workspace`.
 *  - Return value: KDN_OK (0); a negative KDN_ERR_* code when the arguments are
 *    rejected, in which case nothing was enqueued and no device memory was
 *    touched; or a positive hipError_t value when a launch failed.
 *  - NaN or Inf inputs are not checked: they propagate into the outputs.
 *  - Calls that share output or state buffers must be ordered on one stream.
 */
#ifndef KDN_H
#define KDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types of q, k, v, o */
#define KDN_F32 0
#define KDN_BF16 1

/* write modes */
#define KDN_GAIN_DELTA 0 /* b_t = beta_t k_t                                   */
#define KDN_GAIN_DIAG 1  /* diagonal-covariance Kalman gain, cov [B,H,d_k]       */
#define KDN_GAIN_FULL 2  /* full-covariance Kalman gain, cov [B,H,d_k,d_k], d_k <= 64 */
#define KDN_GAIN_ISO 3   /* isotropic Kalman gain: one variance per head, cov [B,H]   */

/* residual forms (PLAIN and NOERASE with the delta write only; the Kalman
 * modes always use the gated form) */
#define KDN_RESID_GATED 0   /* e = v - alpha S^T k                                  */
#define KDN_RESID_PLAIN 1   /* e = v - S^T k                                        */
#define KDN_RESID_NOERASE 2 /* e = v: S = alpha S + beta k v^T (decayed linear attention) */

/* write scores ("A Hippocampus for Linear Attention", sec. 3.3 eq. (6); the
 * two ablation variants of sec. 3.3 "versus recency" and sec. 4.5) */
#define KDN_SCORE_WRITE 0 /* ||b e^T||_F: beta ||e|| (delta), ||g|| ||e|| (Kalman)  */
#define KDN_SCORE_RESID 1 /* ||e|| (the residual alone)                             */
#define KDN_SCORE_VALUE 2 /* beta ||v|| (delta), ||g|| ||v|| (the write strength alone) */

/* cache eviction ("A Hippocampus for Linear Attention", sec. 3.3; sec. 4.5's
 * matched control) */
#define KDN_EVICT_SCORE 0   /* keep the w largest scores (ties: earlier token) */
#define KDN_EVICT_RECENCY 1 /* keep the w most recent tokens                   */

/* status codes */
#define KDN_OK 0
#define KDN_ERR_NULL_POINTER (-1)  /* a required pointer is NULL                   */
#define KDN_ERR_BAD_SHAPE (-2)     /* a size is < 1 (L may be 0) or out of range   */
#define KDN_ERR_BAD_CHUNK (-3)     /* chunk not in {16, 32, 64, 128}                */
#define KDN_ERR_BAD_MODE (-4)      /* unknown mode / residual / score / policy, or a
                                      residual form the write mode does not take   */
#define KDN_ERR_BAD_DTYPE (-5)     /* unknown element type                          */
#define KDN_ERR_UNSUPPORTED (-6)   /* valid but not implemented for these sizes    */
#define KDN_ERR_WORKSPACE (-7)     /* workspace missing or smaller than required   */
#define KDN_ERR_BAD_CAPACITY (-8)  /* cache capacity w not in [1, 256]              */
#define KDN_ERR_BAD_ALIGNMENT (-9) /* a pointer is not 16-byte aligned              */
#define KDN_ERR_SCRATCH_LIMIT (-10) /* needs more than the static scratch array holds */

/* Static, human-readable message for a status code (never NULL). */
const char *kdn_status_string(int status);

/* Library version, major * 10000 + minor * 100 + patch. */
int kdn_version(void);

/*
 * Bytes of device workspace kdn_scan_fwd needs for these arguments: the
 * per-token Kalman gains and covariance maps per chunk (per half chunk for the
 * diagonal write on the matrix-core path) (Kalman modes), on the
 * matrix-core path the per-chunk records of the chunk form ((I + A)^-1 and
 * token scalars), and with with_scores != 0 room for the residuals the write
 * scores are formed from (needed when kdn_scan_fwd is given an `m` output).
 * 0 for the delta write on the float32 path without scores. Pure host
 * computation; 0 for invalid sizes.
 */
size_t kdn_scan_workspace_size(int B, int H, int L, int d_k, int d_v, int chunk,
                               int mode, int in_dtype, int with_scores);

/*
 * Chunkwise-parallel forward scan over a whole sequence (all L tokens of all
 * B*H heads), writing o_t = S_t^T q_t for every token.
 *
 *  q, k      [B,H,L,d_k] in_dtype. The state path assumes unit-norm keys
 *            ("A Hippocampus for Linear Attention", sec. 3.4); the library
 *            does not normalise them.
 *  v         [B,H,L,d_v] in_dtype.
 *  alpha     [B,H,L] float32 decay in (0, 1]; NULL means alpha = 1.
 *  beta      [B,H,L] float32 write strength; required in DELTA mode, ignored
 *            otherwise (the Kalman gain replaces it).
 *  r         [B,H,L] float32 observation-noise variance > 0 (Kalman modes);
 *            NULL means r = 1. Ignored in DELTA mode.
 *  cov_in    prior covariance: [B,H,d_k] (DIAG, entries > 0),
 *            [B,H,d_k,d_k] (FULL, symmetric positive definite) or [B,H] (ISO,
 *            > 0). Required in the Kalman modes, ignored in DELTA mode.
 *  cov_out   final covariance, same shape as cov_in; NULL = not written. May
 *            alias cov_in.
 *  q_noise_var  sigma^2 of the process noise Q_t = (1 - alpha_t^2) sigma^2 (>= 0).
 *  state_in  [B,H,d_k,d_v] float32 initial state; NULL means S_0 = 0.
 *  state_out [B,H,d_k,d_v] float32 final state; NULL = not written. May alias
 *            state_in.
 *  o         [B,H,L,d_v] out_dtype output (bf16 outputs are the float32 result
 *            rounded to nearest even; that rounding alone is up to 2^-9 |o|,
 *            so use float32 output when the error bar is relative to RMS(o)).
 *  m         [B,H,L] float32 write scores, or NULL (not computed): with
 *            score_kind KDN_SCORE_WRITE the norm of each token's rank-one write
 *            ("A Hippocampus for Linear Attention", sec. 3.3 eq. (6)):
 *            beta_t ||e_t|| for the delta write (e_t the residual of the form in
 *            use), ||g_t|| ||e_t|| for the Kalman gains; KDN_SCORE_RESID gives
 *            ||e_t||, KDN_SCORE_VALUE the write strength times ||v_t||. On the
 *            matrix-core path e_t is taken from its fp16 copy (relative error
 *            ~2^-11). Needs the workspace sized with with_scores = 1.
 *  score_kind KDN_SCORE_* (ignored when m is NULL).
 *  chunk     chunk length in tokens: 16, 32, 64 or 128. The result does not
 *            depend on it beyond rounding; L need not be a multiple of it. 128
 *            runs as 64-token chunks (the kernels' largest).
 *  mode      KDN_GAIN_*;  resid  KDN_RESID_* (PLAIN and NOERASE only with
 *            DELTA).
 *  workspace device scratch of at least kdn_scan_workspace_size(...) bytes,
 *            16-byte aligned (may be NULL when that size is 0).
 * Sizes: B, H >= 1; L >= 0 (L = 0 copies state_in to state_out and cov_in to
 * cov_out); 1 <= d_k, d_v <= 128; FULL mode needs d_k <= 64.
 * Paths: bf16 inputs with d_k = 128, d_v a multiple of 32, chunk = 64 (or
 * 128) and 16-byte-aligned q, k, v, o run on the matrix cores: products in
 * fp16 with float32 accumulation, float32 state. The values, the state and the
 * residuals are carried scaled by exact powers of two: a chunk's values once
 * one reaches 2^12, the state once its largest entry reaches 2^11 (checked
 * once per chunk, so it may grow up to 32-fold within one chunk), so they may
 * take any finite magnitude; q and k are staged as fp16 unscaled, so their
 * entries must stay below 65504 (unit keys always do; entries below 2^-14
 * become fp16 subnormals, an absolute error below 2^-24). Every other
 * combination runs the float32 vector path.
 */
int kdn_scan_fwd(const void *q, const void *k, const void *v, int in_dtype,
                 const float *alpha, const float *beta, const float *r,
                 const float *cov_in, float *cov_out, float q_noise_var,
                 const float *state_in, float *state_out,
                 void *o, int out_dtype, float *m, int score_kind,
                 int B, int H, int L, int d_k, int d_v, int chunk, int mode, int resid,
                 void *workspace, size_t workspace_bytes, void *stream);

/* phases of kdn_scan_fwd_phase */
#define KDN_PHASE_ALL 0     /* everything: the same as kdn_scan_fwd                     */
#define KDN_PHASE_PREPARE 1 /* the state-independent part, into the workspace          */
#define KDN_PHASE_STATE 2   /* the sequential state scan that consumes the workspace   */

/*
 * kdn_scan_fwd split in two enqueued parts. PREPARE does everything that does
 * not depend on the state: the covariance recursion and Kalman gains (it
 * writes cov_out) and, on the matrix-core path, the per-chunk inverses
 * (I + A)^-1 of the chunk form; it writes only the workspace and cov_out.
 * STATE then runs the chunk-by-chunk state scan and writes o, m and state_out.
 * A STATE call must see the workspace of a PREPARE call made with the same
 * arguments and inputs (same stream, or ordered by the caller); PREPARE may
 * run ahead on another stream, e.g. for the next batch. Arguments, checks and
 * status codes are those of kdn_scan_fwd; an unknown phase is KDN_ERR_BAD_MODE.
 */
int kdn_scan_fwd_phase(int phase, const void *q, const void *k, const void *v, int in_dtype,
                       const float *alpha, const float *beta, const float *r,
                       const float *cov_in, float *cov_out, float q_noise_var,
                       const float *state_in, float *state_out,
                       void *o, int out_dtype, float *m, int score_kind,
                       int B, int H, int L, int d_k, int d_v, int chunk, int mode, int resid,
                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * kdn_scan_fwd for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation. The
 * arguments are those of kdn_scan_fwd without the workspace; the library uses
 * its own scratch instead: a static device array of KDN_STATIC_SCRATCH_BYTES
 * on every GPU it runs on, held until the process ends. Its device address is
 * looked up once per GPU, on the first call with that GPU current. The call
 * allocates nothing and never synchronises.
 *
 * Limit: a call whose kdn_scan_workspace_size(...) (with_scores = m != NULL)
 * exceeds KDN_STATIC_SCRATCH_BYTES returns KDN_ERR_SCRATCH_LIMIT before
 * anything is enqueued (64 MiB holds, e.g., the delta write at B*H = 64,
 * L = 4096, d = 128 on the matrix-core path). Argument errors are those of
 * kdn_scan_fwd, returned before any HIP call.
 *
 * Sharing: every call on one GPU uses that GPU's one array, which keeps the
 * previous call's contents (no part of a scan needs it cleared). Calls that
 * overlap on one GPU (other streams, other host threads) race on it and give
 * wrong results: order them, e.g. on one stream.
 */
#define KDN_STATIC_SCRATCH_BYTES ((size_t)64 << 20)

int kdn_scan_fwd_static(const void *q, const void *k, const void *v, int in_dtype,
                        const float *alpha, const float *beta, const float *r,
                        const float *cov_in, float *cov_out, float q_noise_var,
                        const float *state_in, float *state_out,
                        void *o, int out_dtype, float *m, int score_kind,
                        int B, int H, int L, int d_k, int d_v, int chunk, int mode, int resid,
                        void *stream);

/*
 * One decode step: the same write and read as kdn_scan_fwd for a single token
 * per head, updating the state (and, in DIAG mode, the covariance) in place.
 * Float32 throughout ("A Hippocampus for Linear Attention", secs. 3.3, 3.5).
 *
 *  q, k      [B,H,d_k] float32;  v [B,H,d_v] float32.
 *  alpha     [B,H] float32 (NULL = 1);  beta [B,H] float32 (DELTA mode).
 *  r         [B,H] float32 (DIAG and ISO modes, NULL = 1).
 *  cov       [B,H,d_k] (DIAG) or [B,H] (ISO) float32, in/out; ignored in DELTA mode.
 *  state     [B,H,d_k,d_v] float32, in/out.
 *  o         [B,H,d_v] float32 out: S_t^T q_t after the write.
 *  m         [B,H] float32 out: the write score of kind score_kind
 *            (KDN_SCORE_*); NULL = not written.
 * Sizes: B, H >= 1; 1 <= d_k, d_v <= 128. Modes DELTA, DIAG and ISO (cov [B,H]).
 */
int kdn_step_decode(const float *q, const float *k, const float *v,
                    const float *alpha, const float *beta, const float *r,
                    float *cov, float q_noise_var, float *state,
                    float *o, float *m, int score_kind,
                    int B, int H, int d_k, int d_v, int mode, int resid, void *stream);

/*
 * HOLA exact cache for one decoding token per head ("A Hippocampus for Linear
 * Attention", sec. 3.3 (top-w cache by write score), sec. 3.4 eq. (7) (read),
 * sec. 3.2 eq. (4) (softmax read)).
 *
 * First the read over the visible set: the cached tokens, the current token
 * and, if sink_logit is given, one null sink (value 0, logit sink_logit[h]):
 *     qn = q / sqrt(mean(q^2) + rms_eps), kn likewise,  l_j = qn . kn_j / sqrt(d_k),
 *     o_cache = sum_j softmax(l)_j v_j.
 * Then the insert: the cache keeps the w tokens with the largest score m
 * (ties: the earlier token). While count < w the token goes to slot `count`;
 * afterwards it replaces the slot with the smallest (m, then largest pos) when
 * its m is strictly larger. Comparisons are on the float32 scores. With
 * policy KDN_EVICT_RECENCY the cache keeps the w most recent tokens instead
 * (a full cache replaces the slot with the smallest pos).
 *
 *  q, k      [B,H,d_k] float32;  v [B,H,d_v] float32;  m [B,H] float32 score.
 *  t         absolute token position (stored in cache_pos; tie-break).
 *  cache_k   [B,H,w,d_k] float32, cache_v [B,H,w,d_v] float32 (exact copies),
 *  cache_m   [B,H,w] float32, cache_pos [B,H,w] int32, cache_count [B,H] int32:
 *            in/out. Start from cache_count = 0.
 *  sink_logit [H] float32 or NULL (no sink).
 *  o_cache   [B,H,d_v] float32 out.
 * Sizes: B, H >= 1; 1 <= d_k, d_v <= 128; 1 <= w <= 256; rms_eps >= 0.
 */
int hola_cache_update(const float *q, const float *k, const float *v, const float *m,
                      int32_t t, float *cache_k, float *cache_v, float *cache_m,
                      int32_t *cache_pos, int32_t *cache_count, const float *sink_logit,
                      float *o_cache, float rms_eps, int B, int H, int d_k, int d_v, int w,
                      int policy, void *stream);

/*
 * Gradients of the delta-write scan (reverse mode) for a loss L with given
 * dL/do (d_o) and dL/dS_L (dstate_out). The pages give no backward pass; the
 * gradient is the adjoint of the token recurrence (c = alpha for the gated
 * residual, 1 for the plain one, 0 without erase):
 *   S_t = (alpha_t I - c_t beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,  o_t = S_t^T q_t,
 *   G_t = dL/dS_t:  G_t += q_t do_t^T,  dq_t = S_t do_t,  y_t = G_t^T k_t,
 *   dv_t = beta_t y_t,  dbeta_t = y_t . e_t,  dk_t = beta_t G_t e_t - c_t beta_t S_{t-1} y_t,
 *   dalpha_t = <G_t, S_{t-1}> - [gated] beta_t y_t . (S_{t-1}^T k_t),
 *   G_{t-1} = alpha_t G_t - c_t beta_t k_t y_t^T,  dS_0 = G_0.
 * The library evaluates it in chunk form (64-token chunks; the same gradient up
 * to rounding order): a forward chain for the chunk-start states, a reverse
 * chain for the state gradients at chunk ends, everything else chunk-parallel
 * on the fp32 matrix cores. Float32 inputs and outputs, layouts as
 * kdn_scan_fwd; the delta write only. The decay gradient is formed as
 * d(log alpha) / alpha, so alpha must be positive (alpha = 0 gives non-finite
 * dalpha).
 *
 *  q, k [B,H,L,d_k], v [B,H,L,d_v], alpha (NULL = 1), beta [B,H,L], state_in
 *            (NULL = 0): the forward call's inputs.
 *  d_o       [B,H,L,d_v];  dstate_out [B,H,d_k,d_v] or NULL (= 0).
 *  dq, dk    [B,H,L,d_k] out;  dv [B,H,L,d_v] out;  dalpha [B,H,L] out
 *            (required when alpha is given, else ignored);  dbeta [B,H,L] out;
 *            dstate_in [B,H,d_k,d_v] out or NULL.
 *  resid     KDN_RESID_GATED, _PLAIN or _NOERASE.
 *  workspace kdn_scan_bwd_workspace_size(...) bytes, 16-byte aligned, device
 *            memory owned by the caller: the state at every chunk start and
 *            the state gradient at every chunk end (B*H*chunks*d_k*d_v floats
 *            each), per-token residuals and their gradients, per-chunk 64 x 64
 *            matrices and [64, d_k] contractions (about 1.2 GB at B=4, H=16,
 *            L=4096, d=128). Its contents need no initialisation.
 * Sizes: B, H >= 1; L >= 0; 1 <= d_k, d_v <= 128; ceil(L / 64) <= 65535.
 */
size_t kdn_scan_bwd_workspace_size(int B, int H, int L, int d_k, int d_v);

int kdn_scan_bwd(const float *q, const float *k, const float *v, const float *alpha,
                 const float *beta, const float *state_in, const float *d_o,
                 const float *dstate_out, float *dq, float *dk, float *dv, float *dalpha,
                 float *dbeta, float *dstate_in, int B, int H, int L, int d_k, int d_v,
                 int resid, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Gradients of every write mode's scan except the full covariance, for float32
 * or bf16 inputs: kdn_scan_bwd extended to the Kalman writes ("Kalman Delta
 * Networks: Uncertainty-aware Associative Memory", abstract: the diagonal and
 * isotropic covariance forms) with the gradients of the observation noise r
 * and of the prior covariance. The loss L has the given dL/do (d_o), dL/dS_L
 * (dstate_out) and, for the Kalman writes, dL/dcov_L (dcov_out).
 *
 * Mode DELTA: as kdn_scan_bwd (resid GATED, PLAIN or NOERASE; beta and dbeta
 * required). Modes DIAG and ISO (resid GATED): the adjoint of the write of
 * kdn_scan_fwd, evaluated as (1) the gains (DIAG) or write strengths (ISO) and
 * the variance before every token, recomputed from cov_in; (2) the chunk-form
 * state backward with those write vectors, which gives dL/d(write vector);
 * (3) the reverse recursion through the gain and covariance maps per token
 * (dp_{t-1} = alpha_t^2 (c_t + e_t dp_t), chunk maps composed in parallel),
 * which adds the gain terms to dk and dalpha and gives dr and dcov_in.
 *
 *  q, k      [B,H,L,d_k] in_dtype (KDN_F32 or KDN_BF16);  v, d_o [B,H,L,d_v] in_dtype
 *            (bf16 operands are converted to float32 inside the library).
 *  alpha, beta, r, cov_in, q_noise_var, state_in: the forward call's inputs
 *            (beta: DELTA only; r (NULL = 1) and cov_in (required): Kalman only).
 *  dstate_out [B,H,d_k,d_v] or NULL (= 0);  dcov_out like cov_in or NULL (= 0).
 *  dq, dk    [B,H,L,d_k] out;  dv [B,H,L,d_v] out;  dalpha [B,H,L] out (required
 *            when alpha is given);  dbeta [B,H,L] out (DELTA);  dr [B,H,L] out
 *            (Kalman, required when r is given);  dcov_in like cov_in, out or NULL;
 *            dstate_in [B,H,d_k,d_v] out or NULL. All outputs float32.
 *  workspace kdn_scan_bwd_ex_workspace_size(B, H, L, d_k, d_v, mode, in_dtype)
 *            bytes, 16-byte aligned; no initialisation needed.
 * Sizes as kdn_scan_bwd. Mode FULL returns KDN_ERR_UNSUPPORTED; alpha must be
 * positive where given (dalpha is formed through log alpha).
 */
size_t kdn_scan_bwd_ex_workspace_size(int B, int H, int L, int d_k, int d_v, int mode,
                                      int in_dtype);

int kdn_scan_bwd_ex(const void *q, const void *k, const void *v, const void *d_o, int in_dtype,
                    const float *alpha, const float *beta, const float *r, const float *cov_in,
                    float q_noise_var, const float *state_in, const float *dstate_out,
                    const float *dcov_out, float *dq, float *dk, float *dv, float *dalpha,
                    float *dbeta, float *dr, float *dcov_in, float *dstate_in, int B, int H,
                    int L, int d_k, int d_v, int mode, int resid, void *workspace,
                    size_t workspace_bytes, void *stream);

/*
 * The HOLA cache over a whole prompt ("A Hippocampus for Linear Attention",
 * sec. 3.3 (top-w cache by write score), sec. 3.4 eq. (7) (visible set: the
 * cache, the causal tokens of the current block and an optional null sink),
 * sec. 3.2 eq. (4)). The L prompt tokens (positions t0 .. t0 + L - 1) are taken
 * in blocks of `block` tokens. Every token of block j reads over the cache as
 * it stood before block j, the tokens of block j up to and including itself,
 * and the sink, with the read of hola_cache_update (RMS-normalised query and
 * keys, 1/sqrt(d_k), softmax). After block j the cache keeps the w best of
 * (cache, block j) by float32 score descending, then position ascending. With
 * block = 1 this is hola_cache_update applied token by token. With policy
 * KDN_EVICT_RECENCY the cache keeps the w most recent tokens (most recent
 * first).
 *
 *  q, k      [B,H,L,d_k] in_dtype (KDN_F32 or KDN_BF16); v [B,H,L,d_v] in_dtype.
 *  m         [B,H,L] float32 write scores of the prompt tokens (e.g. the `m`
 *            output of kdn_scan_fwd). NaN scores rank below every other score.
 *  cache_*   as hola_cache_update: in = the cache before the prompt (count
 *            may be 0), out = after it, slots 0 .. count-1 in rank order.
 *            Cached entries must have positions below t0.
 *  sink_logit [H] float32 or NULL;  o_cache [B,H,L,d_v] float32 out.
 *  workspace device scratch of hola_prefill_workspace_size(...) bytes, 16-byte
 *            aligned.
 * Sizes: B, H >= 1; L >= 0 (L = 0 leaves the cache as it is); 1 <= d_k, d_v
 * <= 128; 1 <= w <= 256; 1 <= block <= 1024; t0 + L <= 2^31 - 1; rms_eps >= 0.
 * The read keeps float32 accuracy: logits and weighted values run on the fp16
 * matrix cores with every float32 operand split into two fp16 parts (three
 * products per float32 product, about 22 significant bits, each part formed
 * from an exact power-of-two multiple of the operand), the softmax on the
 * vector units.
 */
size_t hola_prefill_workspace_size(int B, int H, int L, int d_k, int d_v, int w, int block);

int hola_prefill(const void *q, const void *k, const void *v, int in_dtype, const float *m,
                 int32_t t0, int block, float *cache_k, float *cache_v, float *cache_m,
                 int32_t *cache_pos, int32_t *cache_count, const float *sink_logit,
                 float *o_cache, float rms_eps, int B, int H, int L, int d_k, int d_v, int w,
                 int policy, void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KDN_H */
