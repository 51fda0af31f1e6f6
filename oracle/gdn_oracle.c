/*
 * gdn_oracle.c -- plain sequential CPU oracle of the gated delta-rule layer step.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark may load this library. It shares no code, header, table or
 * helper with the HIP library, and the HIP library never calls it.
 *
 * Everything is computed in IEEE double, one token after another, with no
 * blocking, fusion or reordering beyond what the definitions state. Inputs
 * arrive as doubles that the caller has widened exactly from their storage type.
 *
 * Sources (docs.rs source pages):
 *   [FK] ferrum-kernels 0.8.0, src/backend/metal/vnext_ops/gated_delta_attention_tests.rs
 *        (CPU reference `cpu_segment`, core reference `recurrent_chunk_oracle`,
 *         helpers `normalize_rows`, `sigmoid`, `silu`, `softplus`)
 *   [LM] libmir-metal 0.1.0, src/engine/gated_delta_layer/decode/mod.rs
 *        (`convolve`, `split_qkv`, `precise_gate`)
 *   [FC] ferrox-core 0.24.0, src/gdn.rs
 *        (module doc of the per-token rule, `HeadMap::k_head`, `delta_step`)
 *
 * Readings where the pages leave a step open (each one also listed in the
 * design notes of the repository):
 *   - L2 norm: x * (sum x^2 + eps)^(-1/2) as [FK] `normalize_rows` and the q/k
 *     normalisation inside `cpu_segment` do (eps = 1e-6), not the clamped form of
 *     [FC] `l2_normalize`.
 *   - The read-out scale is applied to the finished dot product (same value as
 *     [FK], which folds it into each term).
 *   - No conv bias (none appears on any page).
 *   - Conv state is [C][K-1], oldest first; w[c][0] multiplies the oldest input.
 *   - No intermediate rounding anywhere; the caller rounds final outputs.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---- scalar activations: [FK] `sigmoid`, `silu`, `softplus` ------------------ */

/* Logistic function, evaluated on the branch that cannot overflow ([FK] `sigmoid`). */
double gdn_oracle_sigmoid(double x)
{
    if (x >= 0.0)
        return 1.0 / (1.0 + exp(-x));
    double e = exp(x);
    return e / (1.0 + e);
}

/* x * sigmoid(x) ([FK] `silu`). */
double gdn_oracle_silu(double x) { return x * gdn_oracle_sigmoid(x); }

/* log(1 + e^x) with the two +-20 cut-overs of [FK] `softplus`. */
double gdn_oracle_softplus(double x)
{
    if (x > 20.0)
        return x;
    if (x < -20.0)
        return exp(x);
    return log1p(exp(x));
}

/* ---- head map: [FC] `HeadMap::k_head`, [FK] GroupedByKeyHead / InterleavedByKeyHead */

/* map 0 = grouped: v-head h reads k-head h / (Hv/Hk).
 * map 1 = tiled (interleaved): v-head h reads k-head h % Hk. */
int gdn_oracle_k_head(int map, int h, int num_k_heads, int num_v_heads)
{
    if (map == 0)
        return h / (num_v_heads / num_k_heads);
    return h % num_k_heads;
}

/* ---- L2 normalisation of one vector ([FK] `normalize_rows`) ------------------ */

void gdn_oracle_l2norm(double *x, int n, double eps)
{
    double ss = 0.0;
    for (int i = 0; i < n; ++i)
        ss += x[i] * x[i];
    double inv = 1.0 / sqrt(ss + eps);
    for (int i = 0; i < n; ++i)
        x[i] *= inv;
}

/* ---- gates ([FK] `cpu_segment`, gate section) -------------------------------
 * decay_kind 0 (log rate):      rate = -exp(decay_param[h])
 * decay_kind 1 (negative rate): rate = decay_param[h]
 * g[t][h]    = rate * softplus(a[t][h] + dt_bias[h])
 * beta[t][h] = sigmoid(b[t][h])                                              */
void gdn_oracle_gates(int T, int Hv, int decay_kind, const double *decay_param,
                      const double *dt_bias, const double *a, const double *b, double *g,
                      double *beta)
{
    for (int t = 0; t < T; ++t)
        for (int h = 0; h < Hv; ++h) {
            double rate = decay_kind == 0 ? -exp(decay_param[h]) : decay_param[h];
            g[(size_t)t * Hv + h] = rate * gdn_oracle_softplus(a[(size_t)t * Hv + h] + dt_bias[h]);
            beta[(size_t)t * Hv + h] = gdn_oracle_sigmoid(b[(size_t)t * Hv + h]);
        }
}

/* ---- depthwise causal conv + SiLU with carried raw inputs -------------------
 * [FK] `cpu_segment` (conv section) and [LM] `convolve`.
 * x     [T][C]   this segment's raw inputs
 * w     [C][K]   taps; w[c][0] meets the oldest input of the window
 * state [C][K-1] raw inputs preceding x, oldest first (updated in place)
 * y     [T][C]   SiLU(sum_m w[c][m] * xhat(t + m - (K-1)))
 * xhat(i) is x[i] for i >= 0, else state[c][(K-1) + i].                        */
void gdn_oracle_conv(int T, int C, int K, const double *x, const double *w, double *state,
                     double *y)
{
    const int W = K - 1;
    double *prev = (double *)malloc(sizeof(double) * (size_t)C * (W > 0 ? W : 1));
    memcpy(prev, state, sizeof(double) * (size_t)C * W);
    for (int t = 0; t < T; ++t)
        for (int c = 0; c < C; ++c) {
            double pre = 0.0;
            for (int m = 0; m < K; ++m) {
                int src = t + m - W;
                double xv = src >= 0 ? x[(size_t)src * C + c] : prev[(size_t)c * W + (W + src)];
                pre += w[(size_t)c * K + m] * xv;
            }
            y[(size_t)t * C + c] = gdn_oracle_silu(pre);
        }
    /* new window = the last K-1 entries of [prev || x] */
    for (int c = 0; c < C; ++c)
        for (int p = 0; p < W; ++p) {
            int src = T + p - W;
            state[(size_t)c * W + p] = src >= 0 ? x[(size_t)src * C + c] : prev[(size_t)c * W + (W + src)];
        }
    free(prev);
}

/* ---- the recurrence ---------------------------------------------------------
 * [FC] module doc and `delta_step`; [FK] `recurrent_chunk_oracle`.
 * For every token t (in order) and v-head h in [h_begin, h_end), with kh the
 * k-head h reads and alpha = exp(g[t][h]), for every value row j:
 *     S[h][j][:] *= alpha
 *     p          = S[h][j][:] . k[t][kh][:]
 *     d          = beta[t][h] * (v[t][h][j] - p)
 *     S[h][j][:] += d * k[t][kh][:]
 *     o[t][h][j]  = scale * (S[h][j][:] . q[t][kh][:])
 * q, k  [T][Hk][dk];  v, o [T][Hv][dv];  g, beta [T][Hv];  S [Hv][dv][dk].     */
void gdn_oracle_recurrence(int T, int Hk, int Hv, int dk, int dv, int map, double scale,
                           const double *q, const double *k, const double *v, const double *g,
                           const double *beta, double *S, double *o, int h_begin, int h_end)
{
    for (int t = 0; t < T; ++t)
        for (int h = h_begin; h < h_end; ++h) {
            int kh = gdn_oracle_k_head(map, h, Hk, Hv);
            const double *kt = k + ((size_t)t * Hk + kh) * dk;
            const double *qt = q + ((size_t)t * Hk + kh) * dk;
            double alpha = exp(g[(size_t)t * Hv + h]);
            double bt = beta[(size_t)t * Hv + h];
            for (int j = 0; j < dv; ++j) {
                double *row = S + ((size_t)h * dv + j) * dk;
                double p = 0.0;
                for (int i = 0; i < dk; ++i) {
                    row[i] *= alpha;
                    p += row[i] * kt[i];
                }
                double d = bt * (v[((size_t)t * Hv + h) * dv + j] - p);
                double r = 0.0;
                for (int i = 0; i < dk; ++i) {
                    row[i] += d * kt[i];
                    r += row[i] * qt[i];
                }
                o[((size_t)t * Hv + h) * dv + j] = scale * r;
            }
        }
}

/* ---- gated RMS norm ([FK] `cpu_segment` output section, [LM] `precise_gate`) --
 * y[r][j] = o[r][j] / sqrt(mean_j o[r][j]^2 + eps) * w[j] * silu(z[r][j])       */
void gdn_oracle_gated_rmsnorm(int rows, int dv, const double *o, const double *z,
                              const double *w, double eps, double *y)
{
    for (int r = 0; r < rows; ++r) {
        const double *orow = o + (size_t)r * dv;
        double ms = 0.0;
        for (int j = 0; j < dv; ++j)
            ms += orow[j] * orow[j];
        double inv = 1.0 / sqrt(ms / dv + eps);
        for (int j = 0; j < dv; ++j)
            y[(size_t)r * dv + j] = orow[j] * inv * w[j] * gdn_oracle_silu(z[(size_t)r * dv + j]);
    }
}

/* ---- one sequence through the core: norm, gates, recurrence, gated norm ------
 * The composition of [FK] `cpu_segment` after its conv. Switches:
 *   l2norm     normalise each (token, k-head) row of q and k
 *   raw_gates  derive g, beta from (a, b, decay_param, dt_bias); else use g, beta
 *   gated_norm apply the gated RMS norm (z, norm_w, norm_eps) to the core output
 * q, k are copied before normalisation; the caller's arrays are not modified.
 * y receives the core output, or the gated-norm output when gated_norm is set. */
typedef struct {
    int T, Hk, Hv, dk, dv, map, decay_kind;
    int l2norm, raw_gates, gated_norm;
    double scale, l2_eps, norm_eps;
    int h_begin, h_end;
} gdn_oracle_core_cfg;

int gdn_oracle_core(const gdn_oracle_core_cfg *cfg, const double *q, const double *k,
                    const double *v, const double *a, const double *b, const double *decay_param,
                    const double *dt_bias, const double *g_in, const double *beta_in,
                    const double *z, const double *norm_w, double *S, double *y)
{
    const int T = cfg->T, Hk = cfg->Hk, Hv = cfg->Hv, dk = cfg->dk, dv = cfg->dv;
    if (T < 0 || Hk <= 0 || Hv <= 0 || Hv % Hk != 0 || dk <= 0 || dv <= 0)
        return 1;
    if (T == 0)
        return 0;
    size_t nqk = (size_t)T * Hk * dk, ng = (size_t)T * Hv, no = (size_t)T * Hv * dv;
    double *qn = (double *)malloc(sizeof(double) * nqk);
    double *kn = (double *)malloc(sizeof(double) * nqk);
    double *g = (double *)malloc(sizeof(double) * ng);
    double *beta = (double *)malloc(sizeof(double) * ng);
    double *o = (double *)malloc(sizeof(double) * no);
    memcpy(qn, q, sizeof(double) * nqk);
    memcpy(kn, k, sizeof(double) * nqk);
    if (cfg->l2norm)
        for (size_t r = 0; r < (size_t)T * Hk; ++r) {
            gdn_oracle_l2norm(qn + r * dk, dk, cfg->l2_eps);
            gdn_oracle_l2norm(kn + r * dk, dk, cfg->l2_eps);
        }
    if (cfg->raw_gates)
        gdn_oracle_gates(T, Hv, cfg->decay_kind, decay_param, dt_bias, a, b, g, beta);
    else {
        memcpy(g, g_in, sizeof(double) * ng);
        memcpy(beta, beta_in, sizeof(double) * ng);
    }
    memset(o, 0, sizeof(double) * no);
    gdn_oracle_recurrence(T, Hk, Hv, dk, dv, cfg->map, cfg->scale, qn, kn, v, g, beta, S, o,
                          cfg->h_begin, cfg->h_end);
    if (cfg->gated_norm)
        gdn_oracle_gated_rmsnorm(T * Hv, dv, o, z, norm_w, cfg->norm_eps, y);
    else
        memcpy(y, o, sizeof(double) * no);
    free(qn);
    free(kn);
    free(g);
    free(beta);
    free(o);
    return 0;
}

/* ---- one sequence through the whole layer: conv, split, core ----------------
 * [FK] `cpu_segment`: conv + SiLU over the mixed [q | k | v] channels, then the
 * split at Hk*dk and 2*Hk*dk ([LM] `split_qkv`), then the core.
 * x [T][QKV] raw mixed inputs; conv_w [QKV][K]; conv_state [QKV][K-1] in/out.  */
int gdn_oracle_segment(const gdn_oracle_core_cfg *cfg, int conv_k, const double *x,
                       const double *conv_w, double *conv_state, const double *a, const double *b,
                       const double *decay_param, const double *dt_bias, const double *z,
                       const double *norm_w, double *S, double *y)
{
    const int T = cfg->T, Hk = cfg->Hk, Hv = cfg->Hv, dk = cfg->dk, dv = cfg->dv;
    const int QK = Hk * dk, QKV = 2 * Hk * dk + Hv * dv;
    if (T < 0 || conv_k < 1)
        return 1;
    double *mixed = (double *)malloc(sizeof(double) * ((size_t)T * QKV + 1));
    gdn_oracle_conv(T, QKV, conv_k, x, conv_w, conv_state, mixed);
    double *q = (double *)malloc(sizeof(double) * ((size_t)T * QK + 1));
    double *k = (double *)malloc(sizeof(double) * ((size_t)T * QK + 1));
    double *v = (double *)malloc(sizeof(double) * ((size_t)T * Hv * dv + 1));
    for (int t = 0; t < T; ++t) {
        const double *row = mixed + (size_t)t * QKV;
        memcpy(q + (size_t)t * QK, row, sizeof(double) * QK);
        memcpy(k + (size_t)t * QK, row + QK, sizeof(double) * QK);
        memcpy(v + (size_t)t * Hv * dv, row + 2 * QK, sizeof(double) * (size_t)Hv * dv);
    }
    int rc = gdn_oracle_core(cfg, q, k, v, a, b, decay_param, dt_bias, NULL, NULL, z, norm_w, S, y);
    free(mixed);
    free(q);
    free(k);
    free(v);
    return rc;
}

/* ---- many independent sequences on host threads (CPU baseline driver) -------
 * Runs gdn_oracle_segment (conv_k > 0) or gdn_oracle_core (conv_k == 0) once per
 * sequence, sequences spread over nthreads POSIX threads. Sequence i has T tokens
 * (all sequences the same length); every per-sequence array is the i-th slice of
 * the batched array. This adds no arithmetic: it only calls the functions above. */
typedef struct {
    const gdn_oracle_core_cfg *cfg;
    int conv_k, batch, nthreads, tid;
    const double *x, *conv_w, *q, *k, *v, *a, *b, *decay_param, *dt_bias, *z, *norm_w;
    double *conv_state, *S, *y;
} batch_job;

static void *batch_worker(void *arg)
{
    batch_job *jb = (batch_job *)arg;
    const gdn_oracle_core_cfg *c = jb->cfg;
    const size_t QKV = 2 * (size_t)c->Hk * c->dk + (size_t)c->Hv * c->dv;
    const size_t T = (size_t)c->T;
    for (int i = jb->tid; i < jb->batch; i += jb->nthreads) {
        const size_t ab = (size_t)i * T * c->Hv, zo = (size_t)i * T * c->Hv * c->dv;
        double *S = jb->S + (size_t)i * c->Hv * c->dv * c->dk;
        if (jb->conv_k > 0)
            gdn_oracle_segment(c, jb->conv_k, jb->x + (size_t)i * T * QKV, jb->conv_w,
                               jb->conv_state + (size_t)i * QKV * (jb->conv_k - 1), jb->a + ab,
                               jb->b + ab, jb->decay_param, jb->dt_bias, jb->z + zo, jb->norm_w, S,
                               jb->y + zo);
        else {
            const size_t qo = (size_t)i * T * c->Hk * c->dk;
            gdn_oracle_core(c, jb->q + qo, jb->k + qo, jb->v + zo, jb->a + ab, jb->b + ab,
                            jb->decay_param, jb->dt_bias, NULL, NULL, jb->z + zo, jb->norm_w, S,
                            jb->y + zo);
        }
    }
    return NULL;
}

int gdn_oracle_batch(const gdn_oracle_core_cfg *cfg, int conv_k, int batch, int nthreads,
                     const double *x, const double *conv_w, double *conv_state, const double *q,
                     const double *k, const double *v, const double *a, const double *b,
                     const double *decay_param, const double *dt_bias, const double *z,
                     const double *norm_w, double *S, double *y)
{
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    pthread_t th[256];
    batch_job jobs[256];
    for (int t = 0; t < nthreads; ++t) {
        batch_job j = {cfg, conv_k, batch, nthreads, t, x, conv_w, q, k, v, a, b,
                       decay_param, dt_bias, z, norm_w, conv_state, S, y};
        jobs[t] = j;
    }
    for (int t = 1; t < nthreads; ++t)
        pthread_create(&th[t], NULL, batch_worker, &jobs[t]);
    batch_worker(&jobs[0]);
    for (int t = 1; t < nthreads; ++t)
        pthread_join(th[t], NULL);
    return 0;
}
