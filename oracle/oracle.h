/*
 * CPU oracle for one greedy decode step of a Llama-style decoder.
 *
 * TEST INFRASTRUCTURE ONLY.  Tests, the package smoke check and the bench's
 * CPU-baseline leg are the only users; the GPU library neither links nor
 * calls it, and it shares no code with the GPU library.
 *
 * Arithmetic is IEEE double throughout (weights are bf16 values widened
 * exactly); the only roundings of the model itself are K and V rows, stored
 * as bf16 (round to nearest even) in the caller's cache.
 *
 * The model is the plain reading of the op list that the page "Megakernels:
 * Deleting the Kernel Boundary to Win Back Microseconds" gives in its sections
 * "Where the microseconds go" (RMS norm, QKV projection, RoPE, attention,
 * output projection, residual add, norm, up and gate projections, SiLU, down
 * projection, residual, LM head) and "One launch, one interpreter" (the same
 * steps as fused opcodes), for the Llama-3.2-1B model that the same page names
 * in its opening paragraph.  The pages never write the equations; the
 * textbook Llama decoder equations are used (see oracle.c for each step).
 */
#ifndef MK_ORACLE_H
#define MK_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab;
    int batch;     /* rows decoded per step */
    int max_seq;   /* cache slots per (layer, K/V, row, group) */
    int tied;      /* 1: LM head weight is the embedding matrix */
    double rms_eps, rope_theta;
    int fp8;       /* 1: every projection matrix and the LM head are used as their FP8
                      quantisation with one scale per matrix (orc_gemv_fp8); 2: with one
                      scale per output row (orc_gemv_fp8_rows); the embedding lookup stays bf16 */
} orc_config;

/* Host pointers, bf16 bit patterns, row-major nn.Linear layout [out][in]. */
typedef struct {
    const uint16_t *embed;      /* [V][H] */
    const uint16_t *final_norm; /* [H] */
    const uint16_t *lm_head;    /* [V][H]; ignored when tied */
    const uint16_t *const *attn_norm; /* L pointers, each [H] */
    const uint16_t *const *wq;        /* [Hq*D][H] */
    const uint16_t *const *wk;        /* [Hkv*D][H] */
    const uint16_t *const *wv;        /* [Hkv*D][H] */
    const uint16_t *const *wo;        /* [H][Hq*D] */
    const uint16_t *const *mlp_norm;  /* [H] */
    const uint16_t *const *w_gate;    /* [F][H] */
    const uint16_t *const *w_up;      /* [F][H] */
    const uint16_t *const *w_down;    /* [H][F] */
} orc_weights;

enum { ORC_OK = 0, ORC_ERR_ARG = -1, ORC_ERR_RANGE = -2, ORC_ERR_NOMEM = -3 };

/* bf16 bit pattern -> exact double. */
double orc_bf16_to_double(uint16_t bits);
/* double -> bf16 bit pattern, round to nearest, ties to even. */
uint16_t orc_bf16_round(double x);

/* out[i] = h[i] * gain[i] / sqrt(mean(h^2) + eps). */
void orc_rmsnorm(const double *h, const uint16_t *gain, int n, double eps, double *out);
/* y[r] = sum_c W[r][c] * x[c]; rows split over `nthreads` threads, each row summed in c order. */
void orc_gemv(const uint16_t *W, int rows, int cols, const double *x, double *y, int nthreads);
/* OCP FP8 E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no
 * infinities, S.1111.111 is NaN): the value of a code. */
double orc_e4m3_to_double(uint8_t code);
/* Code of the E4M3 value nearest to the finite x, ties to the even mantissa;
 * |x| >= 448 gives +-448 (the largest finite value). */
uint8_t orc_e4m3_round(double x);
/* Per-matrix FP8 scale: fp32(amax / 448) with amax the largest |w| of the n
 * bf16 weights (1 when every weight is zero). */
float orc_fp8_scale(const uint16_t *W, size_t n);
/* y[r] = sum_c (s * e4m3(fp32(W[r][c]) / s)) * x[c] with s = orc_fp8_scale(W):
 * the product with the matrix's FP8 quantisation (fp32 division, as the
 * quantiser computes it).  Same threading and summation order as orc_gemv. */
void orc_gemv_fp8(const uint16_t *W, int rows, int cols, const double *x, double *y, int nthreads);
/* The same with one scale per row: s_r = orc_fp8_scale(W[r], cols). */
void orc_gemv_fp8_rows(const uint16_t *W, int rows, int cols, const double *x, double *y, int nthreads);
/* Rotate-half RoPE of one head vector at position `pos`. */
void orc_rope(double *v, int head_dim, int pos, double theta);
/* Softmax attention of one query over n_keys bf16 K/V rows (row stride head_dim). */
void orc_attention(const double *q, const uint16_t *K, const uint16_t *V, int n_keys,
                   int head_dim, double *out);
/* silu(z) = z / (1 + exp(-z)). */
double orc_silu(double z);

/* Bytes of the cache layout bf16 [L][2][B][Hkv][max_seq][D]. */
uint64_t orc_kv_cache_bytes(const orc_config *c);

/*
 * One decode step for every batch row b: token tokens[b] at position
 * positions[b] (0 <= p < max_seq; slots [0, p) of row b must hold earlier K/V).
 * Writes K/V of slot p into kv_cache and logits[b][V] (double).
 * Returns ORC_OK or a negative code (nothing written on argument errors).
 */
int orc_decode_step(const orc_config *c, const orc_weights *w, uint16_t *kv_cache,
                    const int32_t *tokens, const int32_t *positions, double *logits,
                    int nthreads);

/* Index of the largest value, lowest index on ties. */
int orc_argmax(const double *v, int n);

#ifdef __cplusplus
}
#endif
#endif
