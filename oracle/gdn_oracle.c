/*
 * Plain CPU oracle of the Gated DeltaNet (GDN) mixer core: causal depthwise
 * conv + SiLU, L2-normalised q/k, per-value-head gates, the gated delta-rule
 * recurrence on a per-head state S[d_k][d_v], and the gated RMSNorm.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code,
 * header or constant with the HIP library and must never be used as a
 * fallback for it.
 *
 * Everything runs token by token in IEEE double precision, in the order the
 * pages write it.  Sources (page title, item):
 *   [cpu.rs]  "cherenkov qwen4_exp/cpu.rs", fn deltanet and fn causal_conv
 *   [qwen.rs] "oxinfer 0.0.5 src/qwen.rs", DeltaRule::run, Qwen gdn_forward
 *             and the GdnState layout
 *   [exp.rs]  "cortiq-engine 0.6.5 src/qwen4_exp.rs", fn sigmoid / fn silu
 *
 * Readings taken where the pages leave a step open:
 *   - L2 norm is x * (sum x^2 + eps)^(-1/2) with eps = 1e-6 ([qwen.rs] run);
 *     q is further scaled by d_k^(-1/2) ([cpu.rs] deltanet, [qwen.rs] run).
 *   - softplus(x) = x above 20, else log(1 + e^x) ([qwen.rs] run).
 *   - sigmoid / SiLU use the exact exponential ([exp.rs]); the pages' fast
 *     exponential is an approximation of it.
 *   - The gated-norm weight is a plain multiplier of shape [d_v], shared by
 *     all value heads ([qwen.rs] Gdn struct, its norm weight field).
 *   - Value head hv reads key head hv / (H_v / H_k) (contiguous groups,
 *     [cpu.rs] deltanet), or hv mod H_k when the layer uses the tiled order
 *     ([qwen.rs] DeltaRule::run, `tiled`).
 *   - The decay coefficient is -exp(A_log), or a given coefficient for
 *     layers that store it directly ([qwen.rs] weight loading, GGUF ssm_a).
 *   - Kimi Delta Attention ("cortiq-engine 0.8.76 pipeline.rs",
 *     AttnKind::Kda: a per-channel decayed delta rule) is read as the same
 *     rule with the scalar decay replaced by one decay per key channel:
 *     g[i] = coef * softplus(a[i] + dt_bias[i]) for the d_k channels of the
 *     value head, S <- diag(e^g) S, everything else unchanged.  Its
 *     separate q/k/v short convs are the per-channel depthwise conv already
 *     here, and its sigmoid output gate is the sigmoid gate option.
 *   - The conv history holds the last K-1 raw inputs, oldest first, laid out
 *     [K-1][conv_dim] per sequence ([qwen.rs] GdnState).
 *   - A sequence of length 0 passes its state and conv history through.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int32_t h_k, h_v, d_k, d_v, conv_k;
    int32_t gate; /* 0: SiLU output gate, 1: sigmoid output gate */
    double norm_eps, l2_eps;
    int32_t head_map; /* 0: key head hv / (H_v/H_k), 1: key head hv mod H_k */
    int32_t decay_mode; /* 0: one decay per value head, 1: one per key channel */
} oracle_cfg;

/* [exp.rs] fn sigmoid, fn silu; [qwen.rs] DeltaRule::run (softplus). */
static double o_sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }
static double o_silu(double x) { return x * o_sigmoid(x); }
static double o_softplus(double x) { return x > 20.0 ? x : log1p(exp(x)); }

/*
 * One token of the gated delta rule on one value head ([cpu.rs] deltanet,
 * [qwen.rs] DeltaRule::run):
 *   S <- diag(alpha) S;  m = S^T k;  delta = beta (v - m);  S <- S + k delta^T;
 *   o = S^T q  (read out from the updated state).
 * alpha [dk] holds the decay of each key row: all equal to e^g for the
 * scalar-decay rule, one per channel for the per-channel rule.  q and k
 * arrive already normalised (q also scaled).  S is [dk][dv].
 */
static void delta_step(int dk, int dv, const double *q, const double *k,
                       const double *v, const double *alpha, double beta,
                       double *S, double *m, double *delta, double *o)
{
    for (int j = 0; j < dv; ++j) m[j] = 0.0;
    for (int i = 0; i < dk; ++i) {
        double *row = S + (size_t)i * dv;
        for (int j = 0; j < dv; ++j) {
            row[j] *= alpha[i];
            m[j] += row[j] * k[i];
        }
    }
    for (int j = 0; j < dv; ++j) delta[j] = beta * (v[j] - m[j]);
    for (int j = 0; j < dv; ++j) o[j] = 0.0;
    for (int i = 0; i < dk; ++i) {
        double *row = S + (size_t)i * dv;
        for (int j = 0; j < dv; ++j) {
            row[j] += k[i] * delta[j];
            o[j] += row[j] * q[i];
        }
    }
}

/*
 * The delta-rule core alone, for one value head over L tokens.  Inputs are
 * the post-normalisation q [L][dk], k [L][dk], v [L][dv], the log-decay
 * g [L] and write strength beta [L].  S [dk][dv] is updated in place; o
 * [L][dv] receives S_t^T q_t (may be NULL).
 */
void oracle_delta_core(int32_t L, int32_t dk, int32_t dv, const double *q,
                       const double *k, const double *v, const double *g,
                       const double *beta, double *S, double *o)
{
    double *m = malloc(sizeof(double) * dv);
    double *delta = malloc(sizeof(double) * dv);
    double *ot = malloc(sizeof(double) * dv);
    double *alpha = malloc(sizeof(double) * dk);
    for (int t = 0; t < L; ++t) {
        const double a = exp(g[t]);
        for (int i = 0; i < dk; ++i) alpha[i] = a;
        delta_step(dk, dv, q + (size_t)t * dk, k + (size_t)t * dk,
                   v + (size_t)t * dv, alpha, beta[t], S, m, delta, ot);
        if (o) memcpy(o + (size_t)t * dv, ot, sizeof(double) * dv);
    }
    free(m);
    free(delta);
    free(ot);
    free(alpha);
}

/*
 * Causal depthwise conv of one channel at one token ([cpu.rs] causal_conv,
 * [qwen.rs] gdn_forward): h = sum_j w[j] * x~_{t-(K-1)+j}, where the window
 * win[0..K-2] holds the K-1 previous raw inputs oldest first and cur is the
 * raw input at t.  No bias.  Returns silu(h).
 */
static double conv_one(int K, const double *w, const double *win, double cur)
{
    double acc = 0.0;
    for (int j = 0; j < K - 1; ++j) acc += w[j] * win[j];
    acc += w[K - 1] * cur;
    return o_silu(acc);
}

/* Shift the window left by one and append the raw input (oldest first). */
static void conv_push(int K, double *win, double cur)
{
    for (int j = 0; j + 1 < K - 1; ++j) win[j] = win[j + 1];
    if (K > 1) win[K - 2] = cur;
}

/*
 * Standalone conv over packed sequences: x [T][conv_dim] raw inputs,
 * conv_w [conv_dim][K], conv_state [N][K-1][conv_dim] in/out, c
 * [T][conv_dim] = silu(conv).  cu_seqlens [N+1].
 */
void oracle_conv(const oracle_cfg *cfg, int32_t n_seq, const int32_t *cu,
                 const double *conv_w, const double *x, double *conv_state,
                 double *c)
{
    const int K = cfg->conv_k;
    const int CD = 2 * cfg->h_k * cfg->d_k + cfg->h_v * cfg->d_v;
    double *win = malloc(sizeof(double) * (K > 1 ? K - 1 : 1));
    for (int n = 0; n < n_seq; ++n) {
        double *st = conv_state + (size_t)n * (K - 1) * CD;
        for (int ch = 0; ch < CD; ++ch) {
            for (int j = 0; j < K - 1; ++j) win[j] = st[(size_t)j * CD + ch];
            for (int t = cu[n]; t < cu[n + 1]; ++t) {
                double cur = x[(size_t)t * CD + ch];
                c[(size_t)t * CD + ch] =
                    conv_one(K, conv_w + (size_t)ch * K, win, cur);
                conv_push(K, win, cur);
            }
            for (int j = 0; j < K - 1; ++j) st[(size_t)j * CD + ch] = win[j];
        }
    }
    free(win);
}

typedef struct {
    const oracle_cfg *cfg;
    int32_t n_seq;
    const int32_t *cu;
    const double *conv_w, *a_log, *dt_bias, *norm_w;
    const double *decay_coef; /* [H_v] or NULL: then -exp(a_log) */
    const double *qkv, *z, *a, *b;
    const double *conv_in; /* [N][K-1][conv_dim], read only */
    double *S;             /* [N][H_v][dk][dv] in/out */
    double *y;             /* [T][value_dim] */
    double *o_pre;         /* [T][value_dim] or NULL */
    int32_t hv_begin, hv_end;
    int32_t next_task;     /* guarded by lock */
    pthread_mutex_t lock;
} mixer_job;

/*
 * One (sequence, value head) task, token by token: conv + SiLU of the
 * channels this head reads, L2 norm of q and k, gates, one delta-rule step
 * and the gated RMSNorm ([cpu.rs] deltanet, [qwen.rs] gdn_forward).
 */
static void mixer_task(mixer_job *J, int n, int hv)
{
    const oracle_cfg *cfg = J->cfg;
    const int HK = cfg->h_k, HV = cfg->h_v, DK = cfg->d_k, DV = cfg->d_v;
    const int K = cfg->conv_k;
    const int CD = 2 * HK * DK + HV * DV, VD = HV * DV;
    const int hk = cfg->head_map ? hv % HK : hv / (HV / HK);
    const int km1 = K > 1 ? K - 1 : 1;
    /* channel index of each lane: q of hk, k of hk, v of hv */
    const int nch = 2 * DK + DV;
    int *chan = malloc(sizeof(int) * nch);
    for (int i = 0; i < DK; ++i) chan[i] = hk * DK + i;
    for (int i = 0; i < DK; ++i) chan[DK + i] = HK * DK + hk * DK + i;
    for (int i = 0; i < DV; ++i) chan[2 * DK + i] = 2 * HK * DK + hv * DV + i;

    double *win = malloc(sizeof(double) * (size_t)nch * km1);
    double *cq = malloc(sizeof(double) * DK);
    double *ck = malloc(sizeof(double) * DK);
    double *cv = malloc(sizeof(double) * DV);
    double *m = malloc(sizeof(double) * DV);
    double *delta = malloc(sizeof(double) * DV);
    double *o = malloc(sizeof(double) * DV);
    double *alpha = malloc(sizeof(double) * DK);
    double *S = J->S + ((size_t)n * HV + hv) * DK * DV;
    const double *st = J->conv_in + (size_t)n * (K - 1) * CD;

    for (int l = 0; l < nch; ++l)
        for (int j = 0; j < K - 1; ++j)
            win[(size_t)l * km1 + j] = st[(size_t)j * CD + chan[l]];

    const double qscale = 1.0 / sqrt((double)DK);
    const double coef = J->decay_coef ? J->decay_coef[hv] : -exp(J->a_log[hv]);

    for (int t = J->cu[n]; t < J->cu[n + 1]; ++t) {
        const double *xt = J->qkv + (size_t)t * CD;
        for (int l = 0; l < nch; ++l) {
            const double cur = xt[chan[l]];
            const double val = conv_one(K, J->conv_w + (size_t)chan[l] * K,
                                        win + (size_t)l * km1, cur);
            conv_push(K, win + (size_t)l * km1, cur);
            if (l < DK) cq[l] = val;
            else if (l < 2 * DK) ck[l - DK] = val;
            else cv[l - 2 * DK] = val;
        }
        /* L2 normalisation, eps inside the root; q also gets d_k^-1/2. */
        double sq = 0.0, sk = 0.0;
        for (int i = 0; i < DK; ++i) {
            sq += cq[i] * cq[i];
            sk += ck[i] * ck[i];
        }
        const double qinv = 1.0 / sqrt(sq + cfg->l2_eps);
        const double kinv = 1.0 / sqrt(sk + cfg->l2_eps);
        for (int i = 0; i < DK; ++i) {
            cq[i] = cq[i] * qinv * qscale;
            ck[i] = ck[i] * kinv;
        }
        /* Gates: beta = sigmoid(b); g = -exp(A_log) softplus(a + dt_bias),
         * per value head, or per key channel of it (a and dt_bias then hold
         * d_k values per value head). */
        const double beta = o_sigmoid(J->b[(size_t)t * HV + hv]);
        if (cfg->decay_mode) {
            for (int i = 0; i < DK; ++i) {
                const size_t c = (size_t)hv * DK + i;
                alpha[i] = exp(coef * o_softplus(J->a[(size_t)t * HV * DK + c] +
                                                 J->dt_bias[c]));
            }
        } else {
            const double g =
                coef * o_softplus(J->a[(size_t)t * HV + hv] + J->dt_bias[hv]);
            const double ag = exp(g);
            for (int i = 0; i < DK; ++i) alpha[i] = ag;
        }

        delta_step(DK, DV, cq, ck, cv, alpha, beta, S, m, delta, o);

        if (J->o_pre)
            memcpy(J->o_pre + (size_t)t * VD + (size_t)hv * DV, o,
                   sizeof(double) * DV);
        /* Gated RMSNorm: o (mean o^2 + eps)^-1/2 * w * gate(z). */
        double ss = 0.0;
        for (int j = 0; j < DV; ++j) ss += o[j] * o[j];
        const double r = 1.0 / sqrt(ss / DV + cfg->norm_eps);
        double *yt = J->y + (size_t)t * VD + (size_t)hv * DV;
        const double *zt = J->z + (size_t)t * VD + (size_t)hv * DV;
        for (int j = 0; j < DV; ++j) {
            const double gz = cfg->gate ? o_sigmoid(zt[j]) : o_silu(zt[j]);
            yt[j] = o[j] * r * J->norm_w[j] * gz;
        }
    }
    free(alpha);
    free(chan);
    free(win);
    free(cq);
    free(ck);
    free(cv);
    free(m);
    free(delta);
    free(o);
}

static void *mixer_worker(void *arg)
{
    mixer_job *J = arg;
    const int nh = J->hv_end - J->hv_begin;
    const int ntask = J->n_seq * nh;
    for (;;) {
        pthread_mutex_lock(&J->lock);
        const int task = J->next_task++;
        pthread_mutex_unlock(&J->lock);
        if (task >= ntask) break;
        mixer_task(J, task / nh, J->hv_begin + task % nh);
    }
    return NULL;
}

/*
 * The full mixer core over packed sequences.
 *   qkv [T][conv_dim] raw fused projection (channels q | k | v, head-major),
 *   z [T][H_v*d_v], a, b [T][H_v]; conv_w [conv_dim][K]; a_log, dt_bias
 *   [H_v]; norm_w [d_v]; cu [N+1].  With the per-channel decay, a is
 *   [T][H_v*d_k] and dt_bias [H_v*d_k].  decay_coef [H_v], when not NULL,
 *   replaces -exp(a_log) (a_log must then be NULL).
 *   S [N][H_v][d_k][d_v] in/out; conv_state [N][K-1][conv_dim] in/out;
 *   y [T][H_v*d_v] out; o_pre (optional) receives the pre-norm readout.
 * Only value heads [hv_begin, hv_end) run the recurrence (their S, y and
 * o_pre entries are written); the conv history is always advanced for every
 * channel.  Independent (sequence, head) tasks run on nthreads threads; the
 * arithmetic of each task does not depend on the thread count.
 * Returns 0, or -1 on an invalid argument.
 */
int oracle_mixer(const oracle_cfg *cfg, int32_t n_seq, const int32_t *cu,
                 const double *conv_w, const double *a_log,
                 const double *dt_bias, const double *norm_w,
                 const double *decay_coef, const double *qkv, const double *z, const double *a,
                 const double *b, double *S, double *conv_state, double *y,
                 double *o_pre, int32_t hv_begin, int32_t hv_end,
                 int32_t nthreads)
{
    if (cfg->h_k <= 0 || cfg->h_v <= 0 || cfg->h_v % cfg->h_k != 0 ||
        cfg->d_k <= 0 || cfg->d_v <= 0 || cfg->conv_k < 1 || n_seq < 0 ||
        hv_begin < 0 || hv_end > cfg->h_v || hv_begin > hv_end ||
        (cfg->head_map != 0 && cfg->head_map != 1) ||
        (cfg->decay_mode != 0 && cfg->decay_mode != 1) ||
        (a_log == NULL) == (decay_coef == NULL))
        return -1;
    for (int n = 0; n < n_seq; ++n)
        if (cu[n + 1] < cu[n]) return -1;
    const int K = cfg->conv_k;
    const int CD = 2 * cfg->h_k * cfg->d_k + cfg->h_v * cfg->d_v;
    const size_t cs_elems = (size_t)n_seq * (K - 1) * CD;

    /* The tasks read the incoming conv history; keep a copy of it. */
    double *conv_in = malloc(sizeof(double) * (cs_elems ? cs_elems : 1));
    memcpy(conv_in, conv_state, sizeof(double) * cs_elems);

    mixer_job J;
    memset(&J, 0, sizeof(J));
    J.cfg = cfg;
    J.n_seq = n_seq;
    J.cu = cu;
    J.conv_w = conv_w;
    J.a_log = a_log;
    J.dt_bias = dt_bias;
    J.norm_w = norm_w;
    J.decay_coef = decay_coef;
    J.qkv = qkv;
    J.z = z;
    J.a = a;
    J.b = b;
    J.conv_in = conv_in;
    J.S = S;
    J.y = y;
    J.o_pre = o_pre;
    J.hv_begin = hv_begin;
    J.hv_end = hv_end;
    J.next_task = 0;
    pthread_mutex_init(&J.lock, NULL);
    if (nthreads < 1) nthreads = 1;
    if (nthreads == 1) {
        mixer_worker(&J);
    } else {
        pthread_t *th = malloc(sizeof(pthread_t) * nthreads);
        for (int i = 0; i < nthreads; ++i)
            pthread_create(&th[i], NULL, mixer_worker, &J);
        for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
        free(th);
    }
    pthread_mutex_destroy(&J.lock);

    /* New conv history: the last K-1 raw inputs of each sequence, oldest
     * first, reaching back into the old history when L < K-1
     * ([qwen.rs] gdn_forward, conv-state update). */
    for (int n = 0; n < n_seq; ++n) {
        const int L = cu[n + 1] - cu[n];
        for (int s = 0; s < K - 1; ++s) {
            const int tau = L - (K - 1) + s; /* time index within sequence */
            double *dst = conv_state + ((size_t)n * (K - 1) + s) * CD;
            if (tau >= 0)
                memcpy(dst, qkv + (size_t)(cu[n] + tau) * CD,
                       sizeof(double) * CD);
            else
                memcpy(dst, conv_in + ((size_t)n * (K - 1) + (K - 1 + tau)) * CD,
                       sizeof(double) * CD);
        }
    }
    free(conv_in);
    return 0;
}
