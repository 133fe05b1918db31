/*
 * kdn_oracle.c -- plain, slow, sequential float64 reference for the delta-rule
 * family of associative-memory recurrences and the HOLA exact cache.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product library links, loads or
 * calls this file; it is used by the tests, by the package's smoke check and
 * by the benchmark's CPU-baseline leg. It shares no code with the HIP path.
 *
 * Everything is strictly sequential in the token index t, one (batch, head)
 * pair at a time (OpenMP only spreads independent pairs over host threads).
 * Inputs arrive as float32 (the exact values the GPU sees; bf16 inputs are
 * exactly representable in float32) and every operation is done in double.
 *
 * Notation: state S is d_k x d_v, S[i][j] at S[i*dv + j]; the prediction for
 * key k is S^T k (a d_v vector); the read-out is o_t = S_t^T q_t.
 *
 * Sources (page title, then section / equation):
 *  [HOLA]  "A Hippocampus for Linear Attention: An Exact Memory for What the
 *          Recurrent State Forgets", part 2/3: sec. 3.2 eq. (4), sec. 3.3
 *          eqs. (5)-(6), sec. 3.4 eq. (7), sec. 3.5.
 *  [KDN]   "Kalman Delta Networks: Uncertainty-aware Associative Memory",
 *          abstract.
 *  [MBD]   "Memory by Design: Probabilistic Sequence Layers", abstract.
 *  [PC]    "DeltaNet-PC: Test-Time Memory Without Backpropagation Through
 *          Time", summary ("How it works"), eqs. (6)-(7).
 *
 * Readings where the pages leave a step open are listed where they are used
 * (R-numbers match the design notes).
 *
 * Parity pins: every function here is checked in the CPU test-suite against
 * closed forms, brute force and special cases that do not use this file's
 * arithmetic (ridge regression, weighted ridge, exact recall, no-op write,
 * covariance-reset reduction, one-hot keys, softmax attention, sorting).
 * The diagonal-covariance write under stationary process noise with general
 * keys has no closed form: there it is pinned only through its special cases
 * (k = 0, one-hot keys, covariance reset, fixed point), see the tests.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_DELTA 0
#define ORC_DIAG 1
#define ORC_FULL 2
#define ORC_ISO 3
#define ORC_GATED 0
#define ORC_PLAIN 1
#define ORC_NOERASE 2
#define ORC_SCORE_WRITE 0
#define ORC_SCORE_RESID 1
#define ORC_SCORE_VALUE 2
#define ORC_EVICT_SCORE 0
#define ORC_EVICT_RECENCY 1

/*
 * One (batch, head) sequence of the write/read recurrence.
 *
 * Delta write (mode DELTA), gated form [HOLA sec. 3.5, eq. (5)]:
 *     e_t = v_t - alpha_t S_{t-1}^T k_t
 *     S_t = alpha_t S_{t-1} + beta_t k_t e_t^T
 * Plain form (resid PLAIN; no decay inside the residual, as the delta rule is
 * usually written): e_t = v_t - S_{t-1}^T k_t, same update.
 * No-erase form (resid NOERASE): e_t = v_t, i.e. S_t = alpha_t S_{t-1} +
 * beta_t k_t v_t^T, the decayed linear-attention write that the delta rule
 * extends with its erase term [HOLA sec. 3.5; the filter family of MBD
 * abstract].
 *
 * Kalman write (modes DIAG and FULL) [KDN abstract; MBD abstract]: memory is a
 * linear-Gaussian state-space model. Reading R2: v_t = S_t^T k_t + n_t with
 * n_t ~ N(0, r_t I), transition S_t = alpha_t S_{t-1} + w_t. All d_v value
 * columns see the same key and noise, so one d_k x d_k covariance P is shared
 * by every column. Process noise (reading S3): Q_t = (1 - alpha_t^2) sigma^2,
 * a stationary AR(1) prior that pulls uncertainty back to sigma^2 as memory
 * decays (sigma^2 = q_noise_var; 0 gives Q = 0).
 *     predict : S- = alpha S,   P- = alpha^2 P + Q_t I
 *     residual: e  = v - S-^T k                      (the gated residual)
 *     gain    : u = P- k,  s = k^T u + r_t,  b = u / s
 *     update  : S = S- + b e^T,   P = P- - u u^T / s
 * FULL keeps the whole P (the exact Riccati recursion). DIAG keeps only the
 * diagonal p (reading R3/S5, online mean-field projection): the gain uses the
 * exact one-step posterior mean, b = (p- * k) / (sum_i p-_i k_i^2 + r), and the
 * projected posterior keeps the diagonal of the posterior precision,
 * 1/p_i = 1/p-_i + k_i^2 / r, i.e. p_i = p-_i r / (r + p-_i k_i^2).
 * With alpha = 1, r = 1, Q = 0 and P_0 = eps^-1 I the FULL write is the
 * recursive-least-squares update of [PC eq. (7)].
 * ISO keeps one variance p per (batch, head), the isotropic variant that
 * [KDN abstract] lists beside the diagonal one (reading R4): the covariance is
 * p I, the gain is the exact one-step posterior mean under that prior,
 * b = p- k / (p- ||k||^2 + r), and the posterior precision (1/p-) I + k k^T / r
 * is projected back onto multiples of the identity by KL(q||p), which keeps
 * its mean diagonal: 1/p = 1/p- + ||k||^2 / (d_k r).
 *
 * Read-out o_t = S_t^T q_t, after the write (reading S2; the layer output is
 * the predictive mean [MBD abstract]).
 *
 * Score m_t = ||Delta_t||_F with Delta_t = b e^T the token's rank-1 write
 * [HOLA sec. 3.3, eq. (6)]: ||b|| ||e||. In DELTA mode the score is
 * beta_t ||e_t|| exactly as eq. (6) states it (equal to ||b|| ||e|| for unit
 * keys). The page's ablation of the score [HOLA sec. 3.3, "versus recency";
 * sec. 4.5] replaces it by the residual alone (score RESID: ||e_t||) or the
 * write strength alone (score VALUE: beta_t ||v_t||, ||b_t|| ||v_t|| for a
 * Kalman gain).
 */
static void scan_one(int L, int dk, int dv,
                     const float *q, const float *k, const float *v,
                     const float *alpha, const float *beta, const float *r,
                     double *cov, double qvar, double *S,
                     int mode, int resid, int score, double *o, double *m,
                     double *work)
{
    double *e = work;              /* dv */
    double *b = e + dv;            /* dk */
    double *pm = b + dk;           /* dk  (DIAG p-) */
    double *u = pm + dk;           /* dk  (FULL P- k) */
    double *Pm = u + dk;           /* dk*dk (FULL P-) */
    double pm_iso = 0.0, kk_iso = 0.0; /* ISO p- and ||k||^2 */

    for (int t = 0; t < L; ++t) {
        const float *kt = k + (size_t)t * dk;
        const float *qt = q + (size_t)t * dk;
        const float *vt = v + (size_t)t * dv;
        const double a = alpha ? (double)alpha[t] : 1.0;
        const double rt = r ? (double)r[t] : 1.0;
        const double Qt = (1.0 - a * a) * qvar;

        /* predict the covariance */
        if (mode == ORC_DIAG) {
            for (int i = 0; i < dk; ++i) pm[i] = a * a * cov[i] + Qt;
        } else if (mode == ORC_ISO) {
            pm_iso = a * a * cov[0] + Qt;
        } else if (mode == ORC_FULL) {
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dk; ++j)
                    Pm[i * dk + j] = a * a * cov[i * dk + j] + (i == j ? Qt : 0.0);
        }

        /* residual */
        const double scale = (resid == ORC_PLAIN) ? 1.0 : (resid == ORC_NOERASE ? 0.0 : a);
        for (int j = 0; j < dv; ++j) {
            double pred = 0.0;
            for (int i = 0; i < dk; ++i) pred += S[(size_t)i * dv + j] * (double)kt[i];
            e[j] = (double)vt[j] - scale * pred;
        }

        /* write vector */
        double s = 0.0;
        if (mode == ORC_DELTA) {
            const double bt = (double)beta[t];
            for (int i = 0; i < dk; ++i) b[i] = bt * (double)kt[i];
        } else if (mode == ORC_DIAG) {
            s = rt;
            for (int i = 0; i < dk; ++i) s += pm[i] * (double)kt[i] * (double)kt[i];
            for (int i = 0; i < dk; ++i) b[i] = pm[i] * (double)kt[i] / s;
        } else if (mode == ORC_ISO) {
            kk_iso = 0.0;
            for (int i = 0; i < dk; ++i) kk_iso += (double)kt[i] * (double)kt[i];
            s = pm_iso * kk_iso + rt;
            for (int i = 0; i < dk; ++i) b[i] = pm_iso * (double)kt[i] / s;
        } else {
            for (int i = 0; i < dk; ++i) {
                double acc = 0.0;
                for (int j = 0; j < dk; ++j) acc += Pm[i * dk + j] * (double)kt[j];
                u[i] = acc;
            }
            s = rt;
            for (int i = 0; i < dk; ++i) s += (double)kt[i] * u[i];
            for (int i = 0; i < dk; ++i) b[i] = u[i] / s;
        }

        /* state update */
        for (int i = 0; i < dk; ++i)
            for (int j = 0; j < dv; ++j)
                S[(size_t)i * dv + j] = a * S[(size_t)i * dv + j] + b[i] * e[j];

        /* covariance update */
        if (mode == ORC_DIAG) {
            for (int i = 0; i < dk; ++i) {
                const double k2 = (double)kt[i] * (double)kt[i];
                cov[i] = pm[i] * rt / (rt + pm[i] * k2);
            }
        } else if (mode == ORC_ISO) {
            cov[0] = pm_iso * dk * rt / (dk * rt + pm_iso * kk_iso);
        } else if (mode == ORC_FULL) {
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dk; ++j)
                    cov[i * dk + j] = Pm[i * dk + j] - u[i] * u[j] / s;
            /* P is a covariance: symmetric in exact arithmetic. Averaging it with
             * its transpose keeps it so under rounding, whatever the prior. */
            for (int i = 0; i < dk; ++i)
                for (int j = i + 1; j < dk; ++j) {
                    const double avg = 0.5 * (cov[i * dk + j] + cov[j * dk + i]);
                    cov[i * dk + j] = avg;
                    cov[j * dk + i] = avg;
                }
        }

        /* read-out */
        for (int j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int i = 0; i < dk; ++i) acc += S[(size_t)i * dv + j] * (double)qt[i];
            o[(size_t)t * dv + j] = acc;
        }

        /* write-magnitude score */
        if (m) {
            double ee = 0.0, vv = 0.0;
            for (int j = 0; j < dv; ++j) {
                ee += e[j] * e[j];
                vv += (double)vt[j] * (double)vt[j];
            }
            double ws;  /* the write strength */
            if (mode == ORC_DELTA) {
                ws = (double)beta[t];
            } else {
                double bb = 0.0;
                for (int i = 0; i < dk; ++i) bb += b[i] * b[i];
                ws = sqrt(bb);
            }
            m[t] = score == ORC_SCORE_RESID ? sqrt(ee)
                 : score == ORC_SCORE_VALUE ? ws * sqrt(vv)
                                            : ws * sqrt(ee);
        }
    }
}

/*
 * Full scan over [B, H, L, d] inputs.
 *   q, k: [B,H,L,dk] float32; v: [B,H,L,dv] float32.
 *   alpha, beta, r: [B,H,L] float32. alpha NULL => 1; r NULL => 1;
 *   beta is required in DELTA mode and ignored otherwise.
 *   cov: DIAG [B,H,dk] / FULL [B,H,dk,dk] / ISO [B,H] float64, in = prior,
 *        out = final.
 *   S:   [B,H,dk,dv] float64, in = S_0, out = S_L.
 *   o:   [B,H,L,dv] float64 out;  m: [B,H,L] float64 out (may be NULL).
 * Returns 0, or -1 for an unsupported combination.
 */
int oracle_scan(int B, int H, int L, int dk, int dv,
                const float *q, const float *k, const float *v,
                const float *alpha, const float *beta, const float *r,
                double *cov, double q_noise_var, double *S,
                int mode, int resid, int score, double *o, double *m)
{
    if (mode != ORC_DELTA && mode != ORC_DIAG && mode != ORC_FULL && mode != ORC_ISO) return -1;
    if (resid != ORC_GATED && resid != ORC_PLAIN && resid != ORC_NOERASE) return -1;
    if (resid == ORC_PLAIN && mode != ORC_DELTA) return -1;
    if (score < ORC_SCORE_WRITE || score > ORC_SCORE_VALUE) return -1;
    if (mode == ORC_DELTA && !beta) return -1;
    if (mode != ORC_DELTA && !cov) return -1;
    const int BH = B * H;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int bh = 0; bh < BH; ++bh) {
        double *work = (double *)malloc(sizeof(double) * (size_t)(dv + 3 * dk + dk * dk));
        if (!work) {
#pragma omp atomic write
            bad = 1;
            continue;
        }
        const size_t tok = (size_t)bh * L;
        double *covp = NULL;
        if (mode == ORC_DIAG) covp = cov + (size_t)bh * dk;
        if (mode == ORC_FULL) covp = cov + (size_t)bh * dk * dk;
        if (mode == ORC_ISO) covp = cov + bh;
        scan_one(L, dk, dv, q + tok * dk, k + tok * dk, v + tok * dv,
                 alpha ? alpha + tok : NULL, beta ? beta + tok : NULL, r ? r + tok : NULL,
                 covp, q_noise_var, S + (size_t)bh * dk * dv, mode, resid, score,
                 o + tok * dv, m ? m + tok : NULL, work);
        free(work);
    }
    return bad ? -2 : 0;
}

/*
 * Ranking key of a write score. The pages never meet a NaN score; the reading
 * taken here is that a NaN score ranks below every other score (it is ranked
 * as -infinity and stored unchanged), the same rule for one token at a time
 * and for a whole prompt.
 */
static float orc_rank_key(float m) { return m == m ? m : -INFINITY; }

/*
 * HOLA exact cache, one decode token for every (batch, head)
 * [HOLA sec. 3.3 (top-w cache), sec. 3.4 eq. (7) (read), sec. 3.2 eq. (4)].
 *
 * Read first, over the visible set V_t = cache (as it stood before token t)
 * plus the current token itself (the "current block" is one token when
 * decoding), plus one null sink when sink_logit is given (a slot with value 0
 * and logit sink_logit[h]):
 *     qn = q / sqrt(mean(q^2) + eps),  kn_j likewise (RMSNorm with unit gain)
 *     l_j = qn . kn_j / sqrt(dk)
 *     o_cache = sum_j softmax(l)_j v_j
 * Then insert token t with its score m_t. The decision is taken on the score
 * rounded to float32 (reading S10: scores are float32 and ties go to the
 * earlier token). The cache keeps the w tokens with the largest score, ties
 * broken by the smaller position: while it has free slots the token is
 * appended; otherwise it replaces the slot with the smallest (score, then
 * largest position) if and only if its score is strictly larger.
 * Policy RECENCY is the page's matched control [HOLA sec. 4.5]: the cache
 * keeps the w most recent tokens, so a full cache always replaces the slot
 * with the smallest position.
 *
 *   q, k: [B,H,dk] float32; v: [B,H,dv] float32; m: [B,H] float64.
 *   cache_k [B,H,w,dk], cache_v [B,H,w,dv] float32 (exact copies);
 *   cache_m [B,H,w] float32; cache_pos [B,H,w] int32; count [B,H] int32.
 *   sink_logit: [H] float32 or NULL.   o_cache: [B,H,dv] float64 out.
 */
int oracle_hola_step(int B, int H, int dk, int dv, int w,
                     const float *q, const float *k, const float *v, const double *m,
                     int t, float *cache_k, float *cache_v, float *cache_m,
                     int32_t *cache_pos, int32_t *count, const float *sink_logit,
                     double rms_eps, int policy, double *o_cache)
{
    const int BH = B * H;
#pragma omp parallel for schedule(static)
    for (int bh = 0; bh < BH; ++bh) {
        const float *qt = q + (size_t)bh * dk;
        const float *kt = k + (size_t)bh * dk;
        const float *vt = v + (size_t)bh * dv;
        float *ck = cache_k + (size_t)bh * w * dk;
        float *cv = cache_v + (size_t)bh * w * dv;
        float *cm = cache_m + (size_t)bh * w;
        int32_t *cp = cache_pos + (size_t)bh * w;
        const int n = count[bh];
        double *oc = o_cache + (size_t)bh * dv;

        /* RMS-normalised query */
        double qq = 0.0;
        for (int i = 0; i < dk; ++i) qq += (double)qt[i] * qt[i];
        const double qs = 1.0 / sqrt(qq / dk + rms_eps);
        const double inv_sqrt_d = 1.0 / sqrt((double)dk);

        /* logits over the cache slots, then the current token, then the sink */
        double *lg = (double *)malloc(sizeof(double) * (size_t)(n + 2));
        for (int j = 0; j <= n; ++j) {
            const float *kj = (j < n) ? ck + (size_t)j * dk : kt;
            double kk = 0.0, qk = 0.0;
            for (int i = 0; i < dk; ++i) {
                kk += (double)kj[i] * kj[i];
                qk += (double)qt[i] * kj[i];
            }
            const double ks = 1.0 / sqrt(kk / dk + rms_eps);
            lg[j] = qk * qs * ks * inv_sqrt_d;
        }
        int nl = n + 1;
        if (sink_logit) lg[nl++] = (double)sink_logit[bh % H];
        double mx = lg[0];
        for (int j = 1; j < nl; ++j) mx = lg[j] > mx ? lg[j] : mx;
        double den = 0.0;
        for (int j = 0; j < nl; ++j) den += exp(lg[j] - mx);
        for (int c = 0; c < dv; ++c) oc[c] = 0.0;
        for (int j = 0; j <= n; ++j) {   /* the sink's value is 0 */
            const float *vj = (j < n) ? cv + (size_t)j * dv : vt;
            const double p = exp(lg[j] - mx) / den;
            for (int c = 0; c < dv; ++c) oc[c] += p * (double)vj[c];
        }
        free(lg);

        /* top-w insert, decided on the float32 score */
        const float mt = (float)m[bh];
        int slot = -1;
        if (n < w) {
            slot = n;
            count[bh] = n + 1;
        } else if (policy == ORC_EVICT_RECENCY) {
            int oldest = 0;
            for (int j = 1; j < w; ++j) oldest = cp[j] < cp[oldest] ? j : oldest;
            slot = oldest;
        } else {
            int worst = 0;
            for (int j = 1; j < w; ++j) {
                const float kj = orc_rank_key(cm[j]), kw = orc_rank_key(cm[worst]);
                if (kj < kw || (kj == kw && cp[j] > cp[worst])) worst = j;
            }
            if (orc_rank_key(mt) > orc_rank_key(cm[worst])) slot = worst;
        }
        if (slot >= 0) {
            memcpy(ck + (size_t)slot * dk, kt, sizeof(float) * (size_t)dk);
            memcpy(cv + (size_t)slot * dv, vt, sizeof(float) * (size_t)dv);
            cm[slot] = mt;
            cp[slot] = t;
        }
    }
    return 0;
}

/*
 * Gradients of the Kalman writes, modes DIAG and ISO (gated residual), one
 * (batch, head) at a time: the adjoint of the per-token recursion of
 * scan_one, derived by hand and pinned in the tests by finite differences of
 * oracle_scan. Forward, per token (pm = p-, Q = (1 - a^2) sigma^2):
 *   DIAG: pm_i = a^2 p_i + Q,  s = sum_i pm_i k_i^2 + r,  b_i = pm_i k_i / s,
 *         p'_i = pm_i r / D_i,  D_i = r + pm_i k_i^2
 *   ISO : pm = a^2 p + Q,  kk = |k|^2,  s = pm kk + r,  b = (pm / s) k,
 *         p' = pm d r / D,  D = d r + pm kk   (d = d_k)
 *   e = v - a S^T k,  S' = a S + b e^T,  o = S'^T q.
 * Backward, with G = dL/dS' (after adding q do^T) and dp = dL/dp':
 *   dq = S' do,  y = G^T b,  dv = y,  db = G e,
 *   dk = -a S y + (gain terms),  da = <G, S> - y . (S^T k) + (covariance terms),
 *   G <- a G - a k y^T.
 * The gain and covariance terms follow from the chain rule through b and p':
 *   DIAG: ds = -(db . b) / s;  dpm_i = db_i k_i / s + ds k_i^2 + dp_i r^2 / D_i^2;
 *         dk_i += db_i pm_i / s + 2 ds pm_i k_i - 2 dp_i pm_i^2 r k_i / D_i^2;
 *         dr = ds + sum_i dp_i pm_i^2 k_i^2 / D_i^2
 *   ISO : dbeta = db . k;  dk_i += (pm / s) db_i;
 *         dpm = dbeta r / s^2 + dp (d r)^2 / D^2;
 *         dkk = -dbeta pm^2 / s^2 - dp pm^2 d r / D^2;  dk_i += 2 dkk k_i;
 *         dr = -dbeta pm / s^2 + dp pm^2 d kk / D^2
 *   both: dp <- a^2 dpm;  da += 2 a sum dpm (p - sigma^2).
 * At the start dp = dL/dp_L (dcovL, or 0) and G = dL/dS_L (dSL, or 0); at the
 * end dcov0 = dp and dS0 = G. States are recomputed from checkpoints every 64
 * tokens; the covariance before every token is kept.
 *
 *   mode ORC_DIAG (cov [B,H,dk]) or ORC_ISO (cov [B,H]); cov0, dcovL float64;
 *   other inputs as oracle_scan_bwd (r may be NULL = 1; alpha NULL = 1).
 *   outputs float64: dq, dk [B,H,L,dk]; dv [B,H,L,dv]; dalpha, dr [B,H,L];
 *   dcov0 like cov0; dS0 [B,H,dk,dv] (dcov0 and dS0 may be NULL).
 */
int oracle_scan_bwd_kalman(int B, int H, int L, int dk, int dv,
                           const float *q, const float *k, const float *v,
                           const float *alpha, const float *r, const double *cov0,
                           double qvar, const double *S0, const double *d_o,
                           const double *dSL, const double *dcovL, int mode,
                           double *dq, double *dkk, double *dvv, double *dalpha, double *dr,
                           double *dcov0, double *dS0)
{
    if (mode != ORC_DIAG && mode != ORC_ISO) return -1;
    const int CK = 64;
    const int nck = (L + CK - 1) / CK;
    const int BH = B * H;
    const size_t SS = (size_t)dk * dv;
    const int np = mode == ORC_DIAG ? dk : 1;   /* covariance entries per head */
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int bh = 0; bh < BH; ++bh) {
        double *ckpt = (double *)malloc(sizeof(double) * SS * (size_t)(nck + 1));
        double *hist = (double *)malloc(sizeof(double) * SS * (size_t)(CK + 1));
        double *G = (double *)malloc(sizeof(double) * SS);
        double *ph = (double *)malloc(sizeof(double) * (size_t)np * (size_t)(L + 1));
        double *vec = (double *)malloc(sizeof(double) * (size_t)(3 * dv + 5 * dk));
        if (!ckpt || !hist || !G || !ph || !vec) {
#pragma omp atomic write
            bad = 1;
            free(ckpt); free(hist); free(G); free(ph); free(vec);
            continue;
        }
        double *y = vec, *e = y + dv, *pr = e + dv;          /* dv each */
        double *b = pr + dv, *pm = b + dk, *db = pm + dk;    /* dk each */
        double *dpm = db + dk, *dp = dpm + dk;               /* dk each */
        const float *qh = q + (size_t)bh * L * dk, *kh = k + (size_t)bh * L * dk;
        const float *vh = v + (size_t)bh * L * dv;
        const float *ah = alpha ? alpha + (size_t)bh * L : NULL;
        const float *rh = r ? r + (size_t)bh * L : NULL;
        const double *doh = d_o + (size_t)bh * L * dv;

        /* covariance before every token: ph[t * np ..] = p_{t-1} (ph[0] = p_0) */
        for (int i = 0; i < np; ++i) ph[i] = cov0[(size_t)bh * np + i];
        for (int t = 0; t < L; ++t) {
            const double a = ah ? (double)ah[t] : 1.0, rt = rh ? (double)rh[t] : 1.0;
            const double Qt = (1.0 - a * a) * qvar;
            const float *kt = kh + (size_t)t * dk;
            const double *pp = ph + (size_t)t * np;
            double *pn = ph + (size_t)(t + 1) * np;
            if (mode == ORC_DIAG) {
                for (int i = 0; i < dk; ++i) {
                    const double m_ = a * a * pp[i] + Qt, k2 = (double)kt[i] * kt[i];
                    pn[i] = m_ * rt / (rt + m_ * k2);
                }
            } else {
                double kk = 0.0;
                for (int i = 0; i < dk; ++i) kk += (double)kt[i] * kt[i];
                const double m_ = a * a * pp[0] + Qt;
                pn[0] = m_ * dk * rt / (dk * rt + m_ * kk);
            }
        }
        /* the write vector b of token t (and pm, s) from p_{t-1} */
        #define ORC_GAIN(t_, s_out)                                                  \
            do {                                                                     \
                const double a_ = ah ? (double)ah[t_] : 1.0;                         \
                const double r_ = rh ? (double)rh[t_] : 1.0;                         \
                const double Q_ = (1.0 - a_ * a_) * qvar;                            \
                const float *k_ = kh + (size_t)(t_) * dk;                            \
                const double *p_ = ph + (size_t)(t_) * np;                           \
                double s_ = r_;                                                      \
                if (mode == ORC_DIAG) {                                              \
                    for (int i = 0; i < dk; ++i) {                                   \
                        pm[i] = a_ * a_ * p_[i] + Q_;                                \
                        s_ += pm[i] * (double)k_[i] * (double)k_[i];                 \
                    }                                                                \
                    for (int i = 0; i < dk; ++i) b[i] = pm[i] * (double)k_[i] / s_;  \
                } else {                                                             \
                    double kk_ = 0.0;                                                \
                    for (int i = 0; i < dk; ++i) kk_ += (double)k_[i] * k_[i];       \
                    pm[0] = a_ * a_ * p_[0] + Q_;                                    \
                    s_ = pm[0] * kk_ + r_;                                           \
                    for (int i = 0; i < dk; ++i) b[i] = pm[0] * (double)k_[i] / s_;  \
                }                                                                    \
                s_out = s_;                                                          \
            } while (0)

        /* forward: state checkpoints at t = 0, 64, ... (the state before token t) */
        double *S = hist;
        for (size_t i = 0; i < SS; ++i) S[i] = S0 ? S0[(size_t)bh * SS + i] : 0.0;
        for (int t = 0; t < L; ++t) {
            if (t % CK == 0) memcpy(ckpt + SS * (size_t)(t / CK), S, sizeof(double) * SS);
            double s;
            ORC_GAIN(t, s);
            (void)s;
            const double a = ah ? (double)ah[t] : 1.0;
            const float *kt = kh + (size_t)t * dk, *vt = vh + (size_t)t * dv;
            for (int j = 0; j < dv; ++j) {
                double p_ = 0.0;
                for (int i = 0; i < dk; ++i) p_ += S[(size_t)i * dv + j] * (double)kt[i];
                e[j] = (double)vt[j] - a * p_;
            }
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j)
                    S[(size_t)i * dv + j] = a * S[(size_t)i * dv + j] + b[i] * e[j];
        }
        for (size_t i = 0; i < SS; ++i) G[i] = dSL ? dSL[(size_t)bh * SS + i] : 0.0;
        for (int i = 0; i < np; ++i) dp[i] = dcovL ? dcovL[(size_t)bh * np + i] : 0.0;

        for (int ck = nck - 1; ck >= 0; --ck) {
            const int t0 = ck * CK, t1 = (t0 + CK < L) ? t0 + CK : L;
            memcpy(hist, ckpt + SS * (size_t)ck, sizeof(double) * SS);
            for (int t = t0; t < t1; ++t) {
                const double *Sp = hist + SS * (size_t)(t - t0);
                double *Sn = hist + SS * (size_t)(t - t0 + 1);
                double s;
                ORC_GAIN(t, s);
                (void)s;
                const double a = ah ? (double)ah[t] : 1.0;
                const float *kt = kh + (size_t)t * dk, *vt = vh + (size_t)t * dv;
                for (int j = 0; j < dv; ++j) {
                    double p_ = 0.0;
                    for (int i = 0; i < dk; ++i) p_ += Sp[(size_t)i * dv + j] * (double)kt[i];
                    e[j] = (double)vt[j] - a * p_;
                }
                for (int i = 0; i < dk; ++i)
                    for (int j = 0; j < dv; ++j)
                        Sn[(size_t)i * dv + j] = a * Sp[(size_t)i * dv + j] + b[i] * e[j];
            }
            for (int t = t1 - 1; t >= t0; --t) {
                const double *Sp = hist + SS * (size_t)(t - t0);      /* S_{t-1} */
                const double *Sn = hist + SS * (size_t)(t - t0 + 1);  /* S_t */
                double s;
                ORC_GAIN(t, s);
                const double a = ah ? (double)ah[t] : 1.0, rt = rh ? (double)rh[t] : 1.0;
                const float *kt = kh + (size_t)t * dk, *vt = vh + (size_t)t * dv;
                const float *qt = qh + (size_t)t * dk;
                const double *dot = doh + (size_t)t * dv;
                const double *pprev = ph + (size_t)t * np;            /* p_{t-1} */
                const size_t tok = (size_t)bh * L + t;
                for (int i = 0; i < dk; ++i)
                    for (int j = 0; j < dv; ++j) G[(size_t)i * dv + j] += (double)qt[i] * dot[j];
                for (int i = 0; i < dk; ++i) {
                    double acc = 0.0;
                    for (int j = 0; j < dv; ++j) acc += Sn[(size_t)i * dv + j] * dot[j];
                    dq[tok * dk + i] = acc;
                }
                for (int j = 0; j < dv; ++j) {
                    double yy = 0.0, p_ = 0.0;
                    for (int i = 0; i < dk; ++i) {
                        yy += G[(size_t)i * dv + j] * b[i];
                        p_ += Sp[(size_t)i * dv + j] * (double)kt[i];
                    }
                    y[j] = yy;
                    pr[j] = p_;
                    e[j] = (double)vt[j] - a * p_;
                }
                double yp = 0.0, gs = 0.0;
                for (int j = 0; j < dv; ++j) {
                    dvv[tok * dv + j] = y[j];
                    yp += y[j] * pr[j];
                }
                for (size_t i = 0; i < SS; ++i) gs += G[i] * Sp[i];
                double da = gs - yp;
                for (int i = 0; i < dk; ++i) {
                    double ge = 0.0, sy = 0.0;
                    for (int j = 0; j < dv; ++j) {
                        ge += G[(size_t)i * dv + j] * e[j];
                        sy += Sp[(size_t)i * dv + j] * y[j];
                    }
                    db[i] = ge;
                    dkk[tok * dk + i] = -a * sy;
                }
                /* gain and covariance */
                double drt = 0.0;
                if (mode == ORC_DIAG) {
                    double dbb = 0.0;
                    for (int i = 0; i < dk; ++i) dbb += db[i] * b[i];
                    const double ds = -dbb / s;
                    drt = ds;
                    for (int i = 0; i < dk; ++i) {
                        const double ki = (double)kt[i], k2 = ki * ki;
                        const double D = rt + pm[i] * k2, D2 = D * D;
                        dpm[i] = db[i] * ki / s + ds * k2 + dp[i] * rt * rt / D2;
                        dkk[tok * dk + i] += db[i] * pm[i] / s + 2.0 * ds * pm[i] * ki
                                             - 2.0 * dp[i] * pm[i] * pm[i] * rt * ki / D2;
                        drt += dp[i] * pm[i] * pm[i] * k2 / D2;
                    }
                    for (int i = 0; i < dk; ++i) {
                        da += 2.0 * a * dpm[i] * (pprev[i] - qvar);
                        dp[i] = a * a * dpm[i];
                    }
                } else {
                    double kk = 0.0, dbeta = 0.0;
                    for (int i = 0; i < dk; ++i) {
                        kk += (double)kt[i] * kt[i];
                        dbeta += db[i] * (double)kt[i];
                    }
                    const double m_ = pm[0], beta_ = m_ / s, D = dk * rt + m_ * kk, D2 = D * D;
                    const double dpm0 = dbeta * rt / (s * s) + dp[0] * (dk * rt) * (dk * rt) / D2;
                    const double dkk2 = -dbeta * m_ * m_ / (s * s) - dp[0] * m_ * m_ * dk * rt / D2;
                    drt = -dbeta * m_ / (s * s) + dp[0] * m_ * m_ * dk * kk / D2;
                    for (int i = 0; i < dk; ++i)
                        dkk[tok * dk + i] += beta_ * db[i] + 2.0 * dkk2 * (double)kt[i];
                    da += 2.0 * a * dpm0 * (pprev[0] - qvar);
                    dp[0] = a * a * dpm0;
                }
                dalpha[tok] = da;
                dr[tok] = drt;
                for (int i = 0; i < dk; ++i)
                    for (int j = 0; j < dv; ++j)
                        G[(size_t)i * dv + j] = a * G[(size_t)i * dv + j] - a * (double)kt[i] * y[j];
            }
        }
        #undef ORC_GAIN
        if (dS0) memcpy(dS0 + (size_t)bh * SS, G, sizeof(double) * SS);
        if (dcov0) memcpy(dcov0 + (size_t)bh * np, dp, sizeof(double) * (size_t)np);
        free(ckpt); free(hist); free(G); free(ph); free(vec);
    }
    return bad ? -2 : 0;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * HOLA exact cache over a whole prompt, block by block [HOLA sec. 3.3 (top-w
 * cache by write score, order-independent), sec. 3.4 eq. (7) (the visible set:
 * the cache, the causal tokens of the current block and an optional null sink),
 * sec. 3.2 eq. (4) (softmax read)].
 *
 * The L tokens (positions t0 .. t0 + L - 1) are taken in blocks of `block`.
 * For token i of block j the visible set is the cache as it stood before block
 * j, the tokens of block j up to and including i, and the sink. After the
 * whole block has been read, its tokens are inserted: the cache becomes the
 * w best of (cache, block) by score descending, then position ascending, on
 * float32 scores (reading S10). With block = 1 this is the decode step's
 * read-then-insert. On return slots 0 .. count-1 hold the cache in that order.
 * Policy RECENCY keeps the w most recent tokens instead (most recent first).
 *
 *   q, k: [B,H,L,dk] float32; v: [B,H,L,dv] float32; m: [B,H,L] float64.
 *   cache_*: as oracle_hola_step, in = the cache before the prompt, out = after.
 *   o_cache: [B,H,L,dv] float64 out.
 */
typedef struct { float m; int32_t pos; int src; } orc_entry; /* src >= 0: token, < 0: slot -1-src */

static int orc_entry_before(const orc_entry *a, const orc_entry *b, int policy)
{
    if (policy == ORC_EVICT_RECENCY) return a->pos > b->pos;
    const float ka = orc_rank_key(a->m), kb = orc_rank_key(b->m);
    return ka > kb || (ka == kb && a->pos < b->pos);
}

int oracle_hola_prefill(int B, int H, int L, int dk, int dv, int w, int block,
                        const float *q, const float *k, const float *v, const double *m,
                        int t0, float *cache_k, float *cache_v, float *cache_m,
                        int32_t *cache_pos, int32_t *count, const float *sink_logit,
                        double rms_eps, int policy, double *o_cache)
{
    if (block < 1 || w < 1) return -1;
    const int BH = B * H;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int bh = 0; bh < BH; ++bh) {
        const float *qh = q + (size_t)bh * L * dk, *kh = k + (size_t)bh * L * dk;
        const float *vh = v + (size_t)bh * L * dv;
        float *ck = cache_k + (size_t)bh * w * dk, *cv = cache_v + (size_t)bh * w * dv;
        float *cm = cache_m + (size_t)bh * w;
        int32_t *cp = cache_pos + (size_t)bh * w;
        const int n0 = count[bh];
        orc_entry *cur = (orc_entry *)malloc(sizeof(orc_entry) * (size_t)(w + block));
        orc_entry *cand = (orc_entry *)malloc(sizeof(orc_entry) * (size_t)(w + block));
        double *lg = (double *)malloc(sizeof(double) * (size_t)(w + block + 1));
        float *ok = (float *)malloc(sizeof(float) * (size_t)w * (dk + dv));
        if (!cur || !cand || !lg || !ok) {
#pragma omp atomic write
            bad = 1;
            free(cur); free(cand); free(lg); free(ok);
            continue;
        }
        int n = n0;
        for (int s = 0; s < n0; ++s) {
            cur[s].m = cm[s];
            cur[s].pos = cp[s];
            cur[s].src = -1 - s;
        }
        const double inv_sqrt_d = 1.0 / sqrt((double)dk);
        for (int j0 = 0; j0 < L; j0 += block) {
            const int j1 = (j0 + block < L) ? j0 + block : L;
            /* read: every token of the block against cache + causal block tokens */
            for (int i = j0; i < j1; ++i) {
                const float *qt = qh + (size_t)i * dk;
                double qq = 0.0;
                for (int a = 0; a < dk; ++a) qq += (double)qt[a] * qt[a];
                const double qs = 1.0 / sqrt(qq / dk + rms_eps);
                int nl = 0;
                for (int e = 0; e < n + (i - j0 + 1); ++e) {
                    const float *kj;
                    if (e < n) kj = cur[e].src >= 0 ? kh + (size_t)cur[e].src * dk
                                                   : ck + (size_t)(-1 - cur[e].src) * dk;
                    else kj = kh + (size_t)(j0 + e - n) * dk;
                    double kk = 0.0, qk = 0.0;
                    for (int a = 0; a < dk; ++a) {
                        kk += (double)kj[a] * kj[a];
                        qk += (double)qt[a] * kj[a];
                    }
                    lg[nl++] = qk * qs * inv_sqrt_d / sqrt(kk / dk + rms_eps);
                }
                const int nv = nl;
                if (sink_logit) lg[nl++] = (double)sink_logit[bh % H];
                double mx = lg[0];
                for (int e = 1; e < nl; ++e) mx = lg[e] > mx ? lg[e] : mx;
                double den = 0.0;
                for (int e = 0; e < nl; ++e) den += exp(lg[e] - mx);
                double *oc = o_cache + ((size_t)bh * L + i) * dv;
                for (int c = 0; c < dv; ++c) oc[c] = 0.0;
                for (int e = 0; e < nv; ++e) {
                    const float *vj;
                    if (e < n) vj = cur[e].src >= 0 ? vh + (size_t)cur[e].src * dv
                                                   : cv + (size_t)(-1 - cur[e].src) * dv;
                    else vj = vh + (size_t)(j0 + e - n) * dv;
                    const double p = exp(lg[e] - mx) / den;
                    for (int c = 0; c < dv; ++c) oc[c] += p * (double)vj[c];
                }
            }
            /* insert the block: keep the w best of cache + block */
            int nc = 0;
            for (int e = 0; e < n; ++e) cand[nc++] = cur[e];
            for (int i = j0; i < j1; ++i) {
                cand[nc].m = (float)m[(size_t)bh * L + i];
                cand[nc].pos = t0 + i;
                cand[nc].src = i;
                ++nc;
            }
            for (int a = 1; a < nc; ++a) {   /* insertion sort, (m desc, pos asc) */
                orc_entry x = cand[a];
                int b = a - 1;
                while (b >= 0 && orc_entry_before(&x, &cand[b], policy)) {
                    cand[b + 1] = cand[b];
                    --b;
                }
                cand[b + 1] = x;
            }
            n = nc < w ? nc : w;
            for (int e = 0; e < n; ++e) cur[e] = cand[e];
        }
        /* write the final cache back (old slots are read before any is written) */
        for (int e = 0; e < n; ++e) {
            const float *ks = cur[e].src >= 0 ? kh + (size_t)cur[e].src * dk : ck + (size_t)(-1 - cur[e].src) * dk;
            const float *vs = cur[e].src >= 0 ? vh + (size_t)cur[e].src * dv : cv + (size_t)(-1 - cur[e].src) * dv;
            memcpy(ok + (size_t)e * (dk + dv), ks, sizeof(float) * (size_t)dk);
            memcpy(ok + (size_t)e * (dk + dv) + dk, vs, sizeof(float) * (size_t)dv);
        }
        for (int e = 0; e < n; ++e) {
            memcpy(ck + (size_t)e * dk, ok + (size_t)e * (dk + dv), sizeof(float) * (size_t)dk);
            memcpy(cv + (size_t)e * dv, ok + (size_t)e * (dk + dv) + dk, sizeof(float) * (size_t)dv);
            cm[e] = cur[e].m;
            cp[e] = cur[e].pos;
        }
        count[bh] = n;
        free(cur); free(cand); free(lg); free(ok);
    }
    return bad ? -2 : 0;
}

/*
 * Gradients of the delta-write scan (reverse mode), one (batch, head) at a
 * time. The pages give no backward formulas; this is the adjoint of the
 * token recurrence written above, derived by hand and pinned in the tests by
 * finite differences of oracle_scan:
 *
 *   S_t = M_t S_{t-1} + beta_t k_t v_t^T,  M_t = alpha_t I - c_t beta_t k_t k_t^T,
 *   o_t = S_t^T q_t,   e_t = v_t - c_t S_{t-1}^T k_t,
 *   c_t = alpha_t (gated residual), 1 (plain), 0 (no erase).
 *
 * Given dL/do_t and dL/dS_L, with G_t = dL/dS_t accumulated backwards:
 *   G_t += q_t do_t^T;   dq_t = S_t do_t;   y_t = G_t^T k_t;
 *   dv_t = beta_t y_t;   dbeta_t = y_t . e_t;
 *   dk_t = beta_t G_t e_t - c_t beta_t S_{t-1} y_t;
 *   dalpha_t = <G_t, S_{t-1}> - [gated] beta_t y_t . (S_{t-1}^T k_t);
 *   G_{t-1} = alpha_t G_t - c_t beta_t k_t y_t^T;   dS_0 = G_0.
 * States are recomputed from checkpoints every 64 tokens.
 *
 *   inputs as oracle_scan (DELTA mode); d_o [B,H,L,dv]; dS_L [B,H,dk,dv] or NULL;
 *   S0 [B,H,dk,dv] float64 or NULL (= 0).
 *   outputs float64: dq, dk [B,H,L,dk]; dv [B,H,L,dv]; dalpha, dbeta [B,H,L];
 *   dS0 [B,H,dk,dv] (may be NULL).
 */
int oracle_scan_bwd(int B, int H, int L, int dk, int dv,
                    const float *q, const float *k, const float *v,
                    const float *alpha, const float *beta, const double *S0,
                    const double *d_o, const double *dSL, int resid,
                    double *dq, double *dkk, double *dvv, double *dalpha, double *dbeta,
                    double *dS0)
{
    if (resid != ORC_GATED && resid != ORC_PLAIN && resid != ORC_NOERASE) return -1;
    const int CK = 64;
    const int nck = (L + CK - 1) / CK;
    const int BH = B * H;
    const size_t SS = (size_t)dk * dv;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int bh = 0; bh < BH; ++bh) {
        double *ckpt = (double *)malloc(sizeof(double) * SS * (size_t)(nck + 1));
        double *hist = (double *)malloc(sizeof(double) * SS * (size_t)(CK + 1));
        double *G = (double *)malloc(sizeof(double) * SS);
        /* y = G^T k, e = v - c S^T k and p = S^T k are d_v-vectors */
        double *y = (double *)malloc(sizeof(double) * (size_t)(3 * dv));
        if (!ckpt || !hist || !G || !y) {
#pragma omp atomic write
            bad = 1;
            free(ckpt); free(hist); free(G); free(y);
            continue;
        }
        double *e = y + dv, *p = e + dv;
        const float *qh = q + (size_t)bh * L * dk, *kh = k + (size_t)bh * L * dk;
        const float *vh = v + (size_t)bh * L * dv;
        const float *ah = alpha ? alpha + (size_t)bh * L : NULL, *bt = beta + (size_t)bh * L;
        const double *doh = d_o + (size_t)bh * L * dv;
        /* forward: checkpoints at t = 0, 64, 128, ... (the state before token t) */
        double *S = hist;  /* scratch */
        for (size_t i = 0; i < SS; ++i) S[i] = S0 ? S0[(size_t)bh * SS + i] : 0.0;
        for (int t = 0; t < L; ++t) {
            if (t % CK == 0) memcpy(ckpt + SS * (size_t)(t / CK), S, sizeof(double) * SS);
            const double a = ah ? (double)ah[t] : 1.0, b = (double)bt[t];
            const double c = resid == ORC_GATED ? a : (resid == ORC_PLAIN ? 1.0 : 0.0);
            const float *kt = kh + (size_t)t * dk, *vt = vh + (size_t)t * dv;
            for (int j = 0; j < dv; ++j) {
                double pr = 0.0;
                for (int i = 0; i < dk; ++i) pr += S[(size_t)i * dv + j] * (double)kt[i];
                e[j] = (double)vt[j] - c * pr;
            }
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j)
                    S[(size_t)i * dv + j] = a * S[(size_t)i * dv + j] + b * (double)kt[i] * e[j];
        }
        for (size_t i = 0; i < SS; ++i) G[i] = dSL ? dSL[(size_t)bh * SS + i] : 0.0;
        /* backward, chunk by chunk from the end */
        for (int ck = nck - 1; ck >= 0; --ck) {
            const int t0 = ck * CK, t1 = (t0 + CK < L) ? t0 + CK : L;
            /* hist[s] = state before token t0 + s, s = 0 .. t1 - t0 */
            memcpy(hist, ckpt + SS * (size_t)ck, sizeof(double) * SS);
            for (int t = t0; t < t1; ++t) {
                const double *Sp = hist + SS * (size_t)(t - t0);
                double *Sn = hist + SS * (size_t)(t - t0 + 1);
                const double a = ah ? (double)ah[t] : 1.0, b = (double)bt[t];
                const double c = resid == ORC_GATED ? a : (resid == ORC_PLAIN ? 1.0 : 0.0);
                const float *kt = kh + (size_t)t * dk, *vt = vh + (size_t)t * dv;
                for (int j = 0; j < dv; ++j) {
                    double pr = 0.0;
                    for (int i = 0; i < dk; ++i) pr += Sp[(size_t)i * dv + j] * (double)kt[i];
                    e[j] = (double)vt[j] - c * pr;
                }
                for (int i = 0; i < dk; ++i)
                    for (int j = 0; j < dv; ++j)
                        Sn[(size_t)i * dv + j] = a * Sp[(size_t)i * dv + j] + b * (double)kt[i] * e[j];
            }
            for (int t = t1 - 1; t >= t0; --t) {
                const double *Sp = hist + SS * (size_t)(t - t0);      /* S_{t-1} */
                const double *Sn = hist + SS * (size_t)(t - t0 + 1);  /* S_t */
                const double a = ah ? (double)ah[t] : 1.0, b = (double)bt[t];
                const double c = resid == ORC_GATED ? a : (resid == ORC_PLAIN ? 1.0 : 0.0);
                const float *kt = kh + (size_t)t * dk, *vt = vh + (size_t)t * dv;
                const float *qt = qh + (size_t)t * dk;
                const double *dot = doh + (size_t)t * dv;
                const size_t tok = (size_t)bh * L + t;
                for (int i = 0; i < dk; ++i)
                    for (int j = 0; j < dv; ++j) G[(size_t)i * dv + j] += (double)qt[i] * dot[j];
                for (int i = 0; i < dk; ++i) {
                    double s = 0.0;
                    for (int j = 0; j < dv; ++j) s += Sn[(size_t)i * dv + j] * dot[j];
                    dq[tok * dk + i] = s;
                }
                for (int j = 0; j < dv; ++j) {
                    double yy = 0.0, pr = 0.0;
                    for (int i = 0; i < dk; ++i) {
                        yy += G[(size_t)i * dv + j] * (double)kt[i];
                        pr += Sp[(size_t)i * dv + j] * (double)kt[i];
                    }
                    y[j] = yy;
                    p[j] = pr;
                    e[j] = (double)vt[j] - c * pr;
                }
                double db = 0.0, yp = 0.0, gs = 0.0;
                for (int j = 0; j < dv; ++j) {
                    dvv[tok * dv + j] = b * y[j];
                    db += y[j] * e[j];
                    yp += y[j] * p[j];
                }
                for (size_t i = 0; i < SS; ++i) gs += G[i] * Sp[i];
                dbeta[tok] = db;
                dalpha[tok] = gs - (resid == ORC_GATED ? b * yp : 0.0);
                for (int i = 0; i < dk; ++i) {
                    double ge = 0.0, sy = 0.0;
                    for (int j = 0; j < dv; ++j) {
                        ge += G[(size_t)i * dv + j] * e[j];
                        sy += Sp[(size_t)i * dv + j] * y[j];
                    }
                    dkk[tok * dk + i] = b * ge - c * b * sy;
                }
                for (int i = 0; i < dk; ++i)
                    for (int j = 0; j < dv; ++j)
                        G[(size_t)i * dv + j] = a * G[(size_t)i * dv + j] - c * b * (double)kt[i] * y[j];
            }
        }
        if (dS0) memcpy(dS0 + (size_t)bh * SS, G, sizeof(double) * SS);
        free(ckpt); free(hist); free(G); free(y);
    }
    return bad ? -2 : 0;
}
