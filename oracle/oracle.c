/*
 * CPU oracle for one greedy decode step of a Llama-style decoder.
 *
 * TEST INFRASTRUCTURE ONLY: used by tests, the package smoke check and the
 * bench's CPU-baseline timing.  It shares no code with the GPU library.
 *
 * Every step below is the plain definition, in the order the page
 * "Megakernels: Deleting the Kernel Boundary to Win Back Microseconds" lists
 * the ops of one forward pass (section "Where the microseconds go"): RMS norm,
 * QKV projection, RoPE, attention, output projection + residual, norm, up and
 * gate projections, SiLU, down projection + residual, then the LM head.  The
 * page names the model Llama-3.2-1B (opening paragraph) but writes no
 * equations, so the textbook Llama equations are used; where a reading was
 * needed it is stated at the function.  No blocking, fusion, split-KV or
 * chunking: those change only rounding order, never the result.
 *
 * Arithmetic is double; bf16 weights are widened exactly.  K and V are
 * stored in the caller's cache as bf16 (round to nearest even), since the
 * cache is bf16 on both sides.
 */
#include "oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* bf16 is the top half of an IEEE binary32: widen by a 16-bit shift. */
double orc_bf16_to_double(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/*
 * Round a double to the nearest bf16 value (8 significant bits, exponent
 * range of binary32), ties to even, directly from the double (no
 * intermediate float rounding).
 */
uint16_t orc_bf16_round(double x) {
    if (isnan(x)) return 0x7FC0;
    double ax = fabs(x);
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (ax == 0.0) return sign;
    if (isinf(x)) return (uint16_t)(sign | 0x7F80);
    int e;
    frexp(ax, &e);              /* ax = m * 2^e, m in [0.5, 1) */
    int q_exp = e - 8;          /* quantum of an 8-significant-bit value */
    if (q_exp < -133) q_exp = -133; /* bf16 subnormal quantum 2^-133 */
    double q = ldexp(1.0, q_exp);
    double r = nearbyint(ax / q) * q; /* default rounding mode: ties to even */
    if (r > 3.3895313892515355e38) return (uint16_t)(sign | 0x7F80); /* > max bf16 */
    float f = (float)r;         /* exact: r has <= 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(sign | (u >> 16));
}

/* Llama RMSNorm: h * g / sqrt(mean(h^2) + eps). */
void orc_rmsnorm(const double *h, const uint16_t *gain, int n, double eps, double *out) {
    double ss = 0.0;
    for (int i = 0; i < n; ++i) ss += h[i] * h[i];
    double inv = 1.0 / sqrt(ss / n + eps);
    for (int i = 0; i < n; ++i) out[i] = h[i] * inv * orc_bf16_to_double(gain[i]);
}

/*
 * OCP 8-bit floating point E4M3 ("FP8"): sign, 4-bit exponent with bias 7 and
 * 3 mantissa bits; exponent 0 holds the subnormals m * 2^-9; there are no
 * infinities and S.1111.111 is NaN, so the largest finite value is
 * 1.75 * 2^8 = 448.
 */
double orc_e4m3_to_double(uint8_t code) {
    const int s = code >> 7, e = (code >> 3) & 15, m = code & 7;
    if (e == 15 && m == 7) return NAN;
    const double v = e ? ldexp(1.0 + m / 8.0, e - 7) : ldexp((double)m, -9);
    return s ? -v : v;
}

/* Round to the nearest representable value: the spacing of E4M3 values is
 * 2^(e-3) in the binade [2^e, 2^(e+1)) for e >= -6, and 2^-9 below 2^-6. */
uint8_t orc_e4m3_round(double x) {
    const uint8_t sign = signbit(x) ? 0x80 : 0;
    const double a = fabs(x);
    if (a >= 448.0) return sign | 0x7E;
    const int e = a >= ldexp(1.0, -6) ? ilogb(a) : -6;
    const double step = ldexp(1.0, e - 3);
    const double v = nearbyint(a / step) * step; /* a / step is exact; ties to even */
    if (v == 0.0) return sign;
    if (v < ldexp(1.0, -6)) return sign | (uint8_t)(v / ldexp(1.0, -9)); /* subnormal */
    const int E = ilogb(v);
    const int m = (int)((v / ldexp(1.0, E) - 1.0) * 8.0);
    return sign | (uint8_t)(((E + 7) << 3) | m);
}

float orc_fp8_scale(const uint16_t *W, size_t n) {
    double amax = 0.0;
    for (size_t i = 0; i < n; ++i) {
        const double a = fabs(orc_bf16_to_double(W[i]));
        if (a > amax) amax = a;
    }
    if (amax == 0.0) return 1.0f;
    return (float)amax / 448.0f;
}

typedef struct {
    const uint16_t *W;
    int cols;
    const double *x;
    double *y;
    int r0, r1;
    int fp8;
    float scale;
} gemv_job;

static void *gemv_rows(void *p) {
    gemv_job *j = (gemv_job *)p;
    for (int r = j->r0; r < j->r1; ++r) {
        const uint16_t *row = j->W + (size_t)r * j->cols;
        double acc = 0.0;
        if (j->fp8) {
            /* fp8 == 2: every row has its own scale, from its own largest magnitude */
            const float scale = j->fp8 == 2 ? orc_fp8_scale(row, (size_t)j->cols) : j->scale;
            for (int c = 0; c < j->cols; ++c) {
                const float q = (float)orc_bf16_to_double(row[c]) / scale;
                acc += (double)scale * orc_e4m3_to_double(orc_e4m3_round(q)) * j->x[c];
            }
        } else {
            for (int c = 0; c < j->cols; ++c) acc += orc_bf16_to_double(row[c]) * j->x[c];
        }
        j->y[r] = acc;
    }
    return NULL;
}

static void gemv_any(const uint16_t *W, int rows, int cols, const double *x, double *y, int nthreads, int fp8);

/* Matrix-vector product with bf16 weights; the thread split does not change any row's sum. */
void orc_gemv(const uint16_t *W, int rows, int cols, const double *x, double *y, int nthreads) {
    gemv_any(W, rows, cols, x, y, nthreads, 0);
}

void orc_gemv_fp8(const uint16_t *W, int rows, int cols, const double *x, double *y, int nthreads) {
    gemv_any(W, rows, cols, x, y, nthreads, 1);
}

void orc_gemv_fp8_rows(const uint16_t *W, int rows, int cols, const double *x, double *y, int nthreads) {
    gemv_any(W, rows, cols, x, y, nthreads, 2);
}

static void gemv_any(const uint16_t *W, int rows, int cols, const double *x, double *y, int nthreads, int fp8) {
    const float scale = fp8 == 1 ? orc_fp8_scale(W, (size_t)rows * cols) : 1.0f;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nthreads > rows / 64 + 1) nthreads = rows / 64 + 1;
    gemv_job jobs[256];
    pthread_t th[256];
    int launched[256] = {0};
    int per = (rows + nthreads - 1) / nthreads;
    for (int t = 0; t < nthreads; ++t) {
        int r0 = t * per < rows ? t * per : rows;
        int r1 = r0 + per < rows ? r0 + per : rows;
        jobs[t] = (gemv_job){W, cols, x, y, r0, r1, fp8, scale};
    }
    for (int t = 1; t < nthreads; ++t) {
        if (jobs[t].r0 >= jobs[t].r1) continue;
        launched[t] = pthread_create(&th[t], NULL, gemv_rows, &jobs[t]) == 0;
        if (!launched[t]) gemv_rows(&jobs[t]);
    }
    gemv_rows(&jobs[0]);
    for (int t = 1; t < nthreads; ++t)
        if (launched[t]) pthread_join(th[t], NULL);
}

/*
 * Rotary position embedding, rotate-half pairing (i, i + D/2) as in the Llama
 * reference model: frequency theta^(-2i/D), angle pos * freq, both in double.
 *   (u, w) -> (u cos a - w sin a, w cos a + u sin a)
 */
void orc_rope(double *v, int head_dim, int pos, double theta) {
    int half = head_dim / 2;
    for (int i = 0; i < half; ++i) {
        double freq = pow(theta, -2.0 * i / head_dim);
        double a = (double)pos * freq;
        double c = cos(a), s = sin(a);
        double u = v[i], w = v[i + half];
        v[i] = u * c - w * s;
        v[i + half] = w * c + u * s;
    }
}

/*
 * Softmax attention of one query over n_keys cached rows:
 *   s_j = q . K_j / sqrt(D),  p = softmax(s) (max-subtracted),  out = sum_j p_j V_j.
 * The split-KV partials and their log-sum-exp merge that the GPU uses reach
 * this same value (the online-softmax identity mentioned on the page
 * "Megakernels in LLM Inference When Fusion Actually Wins", section "What
 * Defines a Megakernel in Modern Inference"), so the oracle does not split.
 */
void orc_attention(const double *q, const uint16_t *K, const uint16_t *V, int n_keys,
                   int head_dim, double *out) {
    double *s = (double *)malloc(sizeof(double) * (n_keys > 0 ? n_keys : 1));
    double scale = 1.0 / sqrt((double)head_dim);
    double m = -INFINITY;
    for (int j = 0; j < n_keys; ++j) {
        double dot = 0.0;
        for (int d = 0; d < head_dim; ++d) dot += q[d] * orc_bf16_to_double(K[(size_t)j * head_dim + d]);
        s[j] = dot * scale;
        if (s[j] > m) m = s[j];
    }
    double denom = 0.0;
    for (int j = 0; j < n_keys; ++j) {
        s[j] = exp(s[j] - m);
        denom += s[j];
    }
    for (int d = 0; d < head_dim; ++d) out[d] = 0.0;
    for (int j = 0; j < n_keys; ++j) {
        double p = s[j] / denom;
        for (int d = 0; d < head_dim; ++d) out[d] += p * orc_bf16_to_double(V[(size_t)j * head_dim + d]);
    }
    free(s);
}

/* SiLU (swish-1) used by the SwiGLU MLP. */
double orc_silu(double z) { return z / (1.0 + exp(-z)); }

uint64_t orc_kv_cache_bytes(const orc_config *c) {
    return (uint64_t)c->n_layers * 2 * c->batch * c->n_kv_heads * c->max_seq * c->head_dim * 2;
}

/* Start of the bf16 [max_seq][D] block for (layer, kv, row, group). */
static uint16_t *cache_rows(const orc_config *c, uint16_t *kv, int l, int which, int b, int g) {
    size_t idx = (((size_t)l * 2 + which) * c->batch + b) * c->n_kv_heads + g;
    return kv + idx * (size_t)c->max_seq * c->head_dim;
}

int orc_argmax(const double *v, int n) {
    int best = 0;
    for (int i = 1; i < n; ++i)
        if (v[i] > v[best]) best = i;
    return best;
}

static int check_args(const orc_config *c, const orc_weights *w, const uint16_t *kv,
                      const int32_t *tokens, const int32_t *positions, const double *logits) {
    if (!c || !w || !kv || !tokens || !positions || !logits) return ORC_ERR_ARG;
    if (c->n_layers < 1 || c->hidden < 1 || c->n_q_heads < 1 || c->n_kv_heads < 1 ||
        c->head_dim < 2 || c->head_dim % 2 || c->ffn < 1 || c->vocab < 1 || c->batch < 1 ||
        c->max_seq < 1 || c->n_q_heads % c->n_kv_heads)
        return ORC_ERR_ARG;
    if (!w->embed || !w->final_norm || (!c->tied && !w->lm_head)) return ORC_ERR_ARG;
    for (int l = 0; l < c->n_layers; ++l)
        if (!w->attn_norm[l] || !w->wq[l] || !w->wk[l] || !w->wv[l] || !w->wo[l] ||
            !w->mlp_norm[l] || !w->w_gate[l] || !w->w_up[l] || !w->w_down[l])
            return ORC_ERR_ARG;
    for (int b = 0; b < c->batch; ++b) {
        if (tokens[b] < 0 || tokens[b] >= c->vocab) return ORC_ERR_RANGE;
        if (positions[b] < 0 || positions[b] >= c->max_seq) return ORC_ERR_RANGE;
    }
    return ORC_OK;
}

int orc_decode_step(const orc_config *c, const orc_weights *w, uint16_t *kv_cache,
                    const int32_t *tokens, const int32_t *positions, double *logits,
                    int nthreads) {
    int rc = check_args(c, w, kv_cache, tokens, positions, logits);
    if (rc != ORC_OK) return rc;
    const int H = c->hidden, D = c->head_dim, Hq = c->n_q_heads, Hkv = c->n_kv_heads;
    const int F = c->ffn, V = c->vocab, QD = Hq * D, KD = Hkv * D;
    double *h = malloc(sizeof(double) * H), *x = malloc(sizeof(double) * H);
    double *q = malloc(sizeof(double) * QD), *k = malloc(sizeof(double) * KD);
    double *v = malloc(sizeof(double) * KD), *o = malloc(sizeof(double) * QD);
    double *proj = malloc(sizeof(double) * H);
    double *gate = malloc(sizeof(double) * F), *up = malloc(sizeof(double) * F);
    if (!h || !x || !q || !k || !v || !o || !proj || !gate || !up) {
        free(h); free(x); free(q); free(k); free(v); free(o); free(proj); free(gate); free(up);
        return ORC_ERR_NOMEM;
    }
    for (int b = 0; b < c->batch; ++b) {
        const int p = positions[b];
        /* token embedding, no scaling (Llama) */
        const uint16_t *e = w->embed + (size_t)tokens[b] * H;
        for (int i = 0; i < H; ++i) h[i] = orc_bf16_to_double(e[i]);
        for (int l = 0; l < c->n_layers; ++l) {
            /* attention block: RMS norm, Q/K/V projections, RoPE on q and k */
            orc_rmsnorm(h, w->attn_norm[l], H, c->rms_eps, x);
            gemv_any(w->wq[l], QD, H, x, q, nthreads, c->fp8);
            gemv_any(w->wk[l], KD, H, x, k, nthreads, c->fp8);
            gemv_any(w->wv[l], KD, H, x, v, nthreads, c->fp8);
            for (int hd = 0; hd < Hq; ++hd) orc_rope(q + hd * D, D, p, c->rope_theta);
            for (int g = 0; g < Hkv; ++g) orc_rope(k + g * D, D, p, c->rope_theta);
            /* append this position's K and V (bf16) to the cache */
            for (int g = 0; g < Hkv; ++g) {
                uint16_t *Kc = cache_rows(c, kv_cache, l, 0, b, g) + (size_t)p * D;
                uint16_t *Vc = cache_rows(c, kv_cache, l, 1, b, g) + (size_t)p * D;
                for (int d = 0; d < D; ++d) {
                    Kc[d] = orc_bf16_round(k[g * D + d]);
                    Vc[d] = orc_bf16_round(v[g * D + d]);
                }
            }
            /* causal attention over positions 0..p; query head hd reads KV group hd*Hkv/Hq */
            for (int hd = 0; hd < Hq; ++hd) {
                int g = hd * Hkv / Hq;
                orc_attention(q + hd * D, cache_rows(c, kv_cache, l, 0, b, g),
                              cache_rows(c, kv_cache, l, 1, b, g), p + 1, D, o + hd * D);
            }
            /* output projection and residual */
            gemv_any(w->wo[l], H, QD, o, proj, nthreads, c->fp8);
            for (int i = 0; i < H; ++i) h[i] += proj[i];
            /* MLP block: RMS norm, SwiGLU, down projection and residual */
            orc_rmsnorm(h, w->mlp_norm[l], H, c->rms_eps, x);
            gemv_any(w->w_gate[l], F, H, x, gate, nthreads, c->fp8);
            gemv_any(w->w_up[l], F, H, x, up, nthreads, c->fp8);
            for (int i = 0; i < F; ++i) gate[i] = orc_silu(gate[i]) * up[i];
            gemv_any(w->w_down[l], H, F, gate, proj, nthreads, c->fp8);
            for (int i = 0; i < H; ++i) h[i] += proj[i];
        }
        /* final RMS norm and LM head (the embedding matrix when tied) */
        orc_rmsnorm(h, w->final_norm, H, c->rms_eps, x);
        gemv_any(c->tied ? w->embed : w->lm_head, V, H, x, logits + (size_t)b * V, nthreads, c->fp8);
    }
    free(h); free(x); free(q); free(k); free(v); free(o); free(proj); free(gate); free(up);
    return ORC_OK;
}
