/*
 * Oracle for the Qwen3 decoder-block forward pass (see orc.h for the policy).
 * TEST INFRASTRUCTURE ONLY: never linked into the product library.
 *
 * Page titles used in citations:
 *   [P1] "Scalar-Native Qwen3 Reference Runtime As The Numerical Authority"
 *   [P2] "M1 — Load the weights"
 *   [P4] "Portable WebAssembly Runtime Architecture for TinyRustLM"
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -fopenmp (no -march=native).
 */
#include "orc.h"

#include <math.h>
#include <stddef.h>
#include <omp.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------------------------ */
/* Storage conversions                                                                          */
/* ------------------------------------------------------------------------------------------ */

/* bf16 -> f32 is exact: the 16 bits are the top half of the f32 pattern ([P2], weights are kept
 * raw and widened on use). */
float orc_bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* f32 -> bf16, round to nearest, ties to even (the KV cache element type). */
uint16_t orc_f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if (isnan(f)) return (uint16_t)((u >> 16) | 0x40u);
    uint32_t keep = u >> 16;
    uint32_t rest = u & 0xffffu;
    if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u))) keep += 1u;
    return (uint16_t)keep;
}

/* exp evaluated in double, rounded once to f32 (libm-independent to within one rounding). */
float orc_exp(float x) { return (float)exp((double)x); }

static float norm_weight(const void *w, int32_t fmt, int32_t i) {
    return fmt == ORC_FMT_BF16 ? orc_bf16_to_f32(((const uint16_t *)w)[i]) : ((const float *)w)[i];
}

/* ------------------------------------------------------------------------------------------ */
/* Building blocks                                                                              */
/* ------------------------------------------------------------------------------------------ */

/* RMSNorm, [P1] section 2 item 1 (no mean-centering, learned scale): ms = (sum x_i*x_i)/n in
 * index order; inv = 1/sqrt(ms + eps); out_i = w_i * (x_i * inv).  eps sits inside the root and
 * the weight multiplies the normalised value. */
void orc_rmsnorm(const float *x, const float *w, int32_t n, float eps, float *out) {
    float ss = 0.0f;
    for (int32_t i = 0; i < n; ++i) ss = ss + x[i] * x[i];
    float ms = ss / (float)n;
    float inv = 1.0f / sqrtf(ms + eps);
    for (int32_t i = 0; i < n; ++i) out[i] = w[i] * (x[i] * inv);
}

/* RoPE angles, [P1] section 2 item 4: for pair i in [0, d/2): angle = pos * theta^(-2i/d).
 * Angle, cos and sin in double, each rounded once to f32. */
void orc_rope_table(double theta, int32_t head_dim, int32_t pos, float *cos_out, float *sin_out) {
    int32_t half = head_dim / 2;
    for (int32_t i = 0; i < half; ++i) {
        double inv_freq = pow(theta, -2.0 * (double)i / (double)head_dim);
        double a = (double)pos * inv_freq;
        cos_out[i] = (float)cos(a);
        sin_out[i] = (float)sin(a);
    }
}

/* Rotation of pairs (i, i + d/2) of one head:
 *   v'_i       = v_i * c_i - v_{i+d/2} * s_i
 *   v'_{i+d/2} = v_{i+d/2} * c_i + v_i * s_i                                                */
void orc_rope_apply(float *v, int32_t head_dim, const float *cos_t, const float *sin_t) {
    int32_t half = head_dim / 2;
    for (int32_t i = 0; i < half; ++i) {
        float a = v[i], b = v[i + half];
        v[i] = a * cos_t[i] - b * sin_t[i];
        v[i + half] = b * cos_t[i] + a * sin_t[i];
    }
}

/* Stable softmax, [P1] section 7 "Logit Softmax Stability" and [P4] "Stable softmax":
 * m = max s; e_i = exp(s_i - m); z = sum e_i in order; p_i = e_i / z.
 * n == 0 is an error; n == 1 gives exactly 1 with no exponential; a NaN score or z that is not
 * finite and positive is a numerical failure. */
int32_t orc_softmax(const float *s, int32_t n, float *p) {
    if (n <= 0) return ORC_INVALID_ARGUMENT;
    for (int32_t i = 0; i < n; ++i)
        if (isnan(s[i])) return ORC_NUMERICAL_FAILURE;
    if (n == 1) {
        p[0] = 1.0f;
        return ORC_OK;
    }
    float m = s[0];
    for (int32_t i = 1; i < n; ++i)
        if (s[i] > m) m = s[i];
    float z = 0.0f;
    for (int32_t i = 0; i < n; ++i) {
        p[i] = orc_exp(s[i] - m);
        z = z + p[i];
    }
    if (!(z > 0.0f) || isinf(z)) return ORC_NUMERICAL_FAILURE;
    for (int32_t i = 0; i < n; ++i) p[i] = p[i] / z;
    return ORC_OK;
}

/* Scaled dot-product attention of one query head over n cached positions, [P1] section 2 item 5:
 * s_j = (sum_d q_d * K_jd) * f32(1/sqrt(d)); p = softmax(s); out_d = sum_j p_j * V_jd in order.
 * K and V are the cached values (bf16-rounded values widened exactly to f32 in the default mode). */
int32_t orc_attention_head(const float *q, const float *k_rows, const float *v_rows, int32_t n, int32_t head_dim,
                           float *out) {
    if (n <= 0) return ORC_INVALID_ARGUMENT;
    float scale = (float)(1.0 / sqrt((double)head_dim));
    float *s = (float *)malloc(sizeof(float) * (size_t)n * 2);
    if (!s) return ORC_INVALID_ARGUMENT;
    float *p = s + n;
    for (int32_t j = 0; j < n; ++j) {
        float dot = 0.0f;
        for (int32_t d = 0; d < head_dim; ++d)
            dot = dot + q[d] * k_rows[(size_t)j * head_dim + d];
        s[j] = dot * scale;
    }
    int32_t rc = orc_softmax(s, n, p);
    if (rc == ORC_OK) {
        for (int32_t d = 0; d < head_dim; ++d) {
            float acc = 0.0f;
            for (int32_t j = 0; j < n; ++j) acc = acc + p[j] * v_rows[(size_t)j * head_dim + d];
            out[d] = acc;
        }
    }
    free(s);
    return rc;
}

/* Grouped-query attention, [P1] section 2 item 5 and [P4] "Shape invariants": with
 * g = n_q / n_kv, query head h reads KV head floor(h / g).  k_heads / v_heads point at head 0 of a
 * [head][pos][dim] block whose heads are head_stride floats apart; n positions are visible (the
 * causal mask of a token at position n-1).  Heads are independent, so they may run on separate
 * threads without changing any sum. */
int32_t orc_gqa_attention(const float *q, int32_t n_q, int32_t n_kv, const float *k_heads, const float *v_heads,
                          size_t head_stride, int32_t n, int32_t head_dim, float *out) {
    if (n_q <= 0 || n_kv <= 0 || n_q % n_kv) return ORC_INVALID_ARGUMENT;
    int32_t group = n_q / n_kv;
    int32_t rc = ORC_OK;
#pragma omp parallel for schedule(static)
    for (int32_t h = 0; h < n_q; ++h) {
        int32_t kvh = h / group;
        int32_t r = orc_attention_head(q + (size_t)h * head_dim, k_heads + (size_t)kvh * head_stride,
                                       v_heads + (size_t)kvh * head_stride, n, head_dim, out + (size_t)h * head_dim);
        if (r != ORC_OK) {
#pragma omp critical
            rc = r;
        }
    }
    return rc;
}

/* SiLU(z) = z * sigma(z) with sigma(z) = 1 / (1 + exp(-z)), [P1] section 5 (MLP step). */
float orc_silu(float z) {
    float sig = 1.0f / (1.0f + orc_exp(-z));
    return z * sig;
}

/* Q8 dot, [P1] section 3 "The Q8_0 Block Contract" and section 5 "Quantized Tensor Access":
 * per block the scale is taken as f32, each code is promoted to f32, and
 * acc = acc + act_i * (q_i * scale) runs strictly from index 0 upward.  Scales here are f32 (one
 * per 32 codes along the input dimension). */
float orc_q8_dot(const int8_t *codes, const float *scales, const float *act, int32_t n) {
    float acc = 0.0f;
    for (int32_t b = 0; b < n / 32; ++b) {
        float scale = scales[b];
        for (int32_t i = 0; i < 32; ++i) {
            float q = (float)codes[b * 32 + i];
            acc = acc + act[b * 32 + i] * (q * scale);
        }
    }
    return acc;
}

/* IEEE 754 binary16 -> f32, from the format's definition: sign bit, 5-bit exponent (bias 15), 10-bit
 * fraction; exponent 0 is a subnormal m * 2^-24, exponent 31 an infinity (m = 0) or a NaN.  Every binary16
 * value is exactly representable in f32, so no rounding happens. */
float orc_f16_to_f32(uint16_t h) {
    const uint32_t sign = h >> 15, e = (h >> 10) & 0x1fu, m = h & 0x3ffu;
    float v;
    if (e == 0) v = (float)m * 0x1p-24f;
    else if (e == 31) v = m ? NAN : INFINITY;
    else v = ldexpf((float)(1024u + m), (int)e - 25);
    return sign ? -v : v;
}

/* Q8_0 dot, [P1] section 3 "The Q8_0 Block Contract" and section 5 "Quantized Tensor Access": a row is a
 * run of 34-byte blocks; per block the little-endian f16 scale is read and promoted to f32, each signed
 * 8-bit code is promoted to f32, and acc = acc + act_i * (q_i * scale) runs strictly from index 0 upward. */
float orc_q8_0_dot(const uint8_t *blocks, const float *act, int32_t n) {
    float acc = 0.0f;
    for (int32_t b = 0; b < n / 32; ++b) {
        const uint8_t *blk = blocks + (size_t)b * 34;
        const float scale = orc_f16_to_f32((uint16_t)(blk[0] | (blk[1] << 8)));
        for (int32_t i = 0; i < 32; ++i) {
            const float q = (float)(int8_t)blk[2 + i];
            acc = acc + act[b * 32 + i] * (q * scale);
        }
    }
    return acc;
}

/* Dynamic int8 quantization of an activation vector, per block of 32 ([P3] section 5 "Q8_0 Mixed-Precision
 * Matrix Multiplication": the f32 activations are quantized to the Q8_0 form per row before the dot, the
 * integers bounded to [-127, 127]): d = max|x| / 127 over the block (f32 division), q = x / d rounded to
 * nearest with ties away from zero and clamped to [-127, 127].  A block with d = 0 gets zero codes; a block
 * whose d is not finite (a NaN or infinite input) gets zero codes and keeps d, so the non-finite value
 * reaches the dot product instead of being repaired. */
void orc_quantize_act8(const float *x, int32_t n, int8_t *q, float *d) {
    for (int32_t b = 0; b < n / 32; ++b) {
        float amax = 0.0f;
        for (int32_t i = 0; i < 32; ++i) {
            const float a = fabsf(x[b * 32 + i]);
            if (isnan(a)) { /* a NaN makes the block's scale NaN */
                amax = a;
                break;
            }
            if (a > amax) amax = a;
        }
        const float db = amax / 127.0f;
        d[b] = db;
        for (int32_t i = 0; i < 32; ++i) {
            float v = 0.0f;
            if (db > 0.0f && isfinite(db)) {
                v = roundf(x[b * 32 + i] / db);
                if (v > 127.0f) v = 127.0f;
                if (v < -127.0f) v = -127.0f;
            }
            q[b * 32 + i] = (int8_t)v;
        }
    }
}

/* q8 x q8 dot ([P3] section 5 "Floating Reduction Order"; [P4] "SIMD128 q8 design"): per block the 32
 * products of int8 weight and activation codes are summed in int32 -- at most 32 * 127 * 127 = 516,128 in
 * magnitude, inside the [P4] "Integer-overflow rule" bound 2^31 - 1 -- then converted to f32 and multiplied by
 * the product of the two block scales, acc = acc + f32(isum) * (ws * da), blocks in order. */
float orc_q8q8_dot(const int8_t *wq, const float *ws, const int8_t *aq, const float *ad, int32_t n) {
    float acc = 0.0f;
    for (int32_t b = 0; b < n / 32; ++b) {
        int32_t isum = 0;
        for (int32_t i = 0; i < 32; ++i) isum += (int32_t)wq[b * 32 + i] * (int32_t)aq[b * 32 + i];
        acc = acc + (float)isum * (ws[b] * ad[b]);
    }
    return acc;
}

/* y = W x with x quantized to int8 per block first (Q8 weights, q8 x q8 dots). */
static void matvec_act8(const orc_mat_t *m, const float *x, float *out) {
    int8_t *q = (int8_t *)malloc((size_t)m->cols);
    float *d = (float *)malloc(sizeof(float) * (size_t)(m->cols / 32));
    orc_quantize_act8(x, m->cols, q, d);
#pragma omp parallel for schedule(static)
    for (int32_t r = 0; r < m->rows; ++r)
        out[r] = orc_q8q8_dot(m->codes + (size_t)r * m->cols, m->scales + (size_t)r * (m->cols / 32), q, d, m->cols);
    free(q);
    free(d);
}

/* bf16 weight row dot: acc = acc + act_i * w_i in index order, w_i widened exactly. */
float orc_bf16_dot(const uint16_t *w, const float *act, int32_t n) {
    float acc = 0.0f;
    for (int32_t i = 0; i < n; ++i) acc = acc + act[i] * orc_bf16_to_f32(w[i]);
    return acc;
}

/* Dequantized weight: one f32 multiply q * scale for Q8, exact widening for bf16. */
void orc_dequant_row(const orc_mat_t *m, int32_t row, float *out) {
    size_t base = (size_t)row * (size_t)m->cols;
    if (m->q8_0) {
        const uint8_t *blocks = m->q8_0 + (size_t)row * (size_t)(m->cols / 32) * 34;
        for (int32_t i = 0; i < m->cols; ++i) {
            const uint8_t *blk = blocks + (size_t)(i / 32) * 34;
            out[i] = (float)(int8_t)blk[2 + i % 32] * orc_f16_to_f32((uint16_t)(blk[0] | (blk[1] << 8)));
        }
        return;
    }
    for (int32_t i = 0; i < m->cols; ++i) {
        if (m->bf16)
            out[i] = orc_bf16_to_f32(m->bf16[base + i]);
        else
            out[i] = (float)m->codes[base + i] * m->scales[(size_t)row * (m->cols / 32) + i / 32];
    }
}

static float row_dot(const orc_mat_t *m, int32_t row, const float *x) {
    size_t base = (size_t)row * (size_t)m->cols;
    if (m->bf16) return orc_bf16_dot(m->bf16 + base, x, m->cols);
    if (m->q8_0) return orc_q8_0_dot(m->q8_0 + (size_t)row * (size_t)(m->cols / 32) * 34, x, m->cols);
    return orc_q8_dot(m->codes + base, m->scales + (size_t)row * (m->cols / 32), x, m->cols);
}

/* y = W x for a canonical [out, in] matrix (y = x W^T, [P2] "weights are stored [out, in]"). */
void orc_matvec(const orc_mat_t *m, const float *x, float *out) {
#pragma omp parallel for schedule(static)
    for (int32_t r = 0; r < m->rows; ++r) out[r] = row_dot(m, r, x);
}

/* Greedy choice, [P4] "Sampling order" (temperature 0): the greatest value, lowest index on ties.
 * Any non-finite value is a numerical failure ([P1] section 4, NaN/Inf rejection). */
int32_t orc_argmax(const float *v, int32_t n, int32_t *idx) {
    int32_t best = 0;
    for (int32_t i = 0; i < n; ++i) {
        if (!isfinite(v[i])) return ORC_NUMERICAL_FAILURE;
        if (v[i] > v[best]) best = i;
    }
    *idx = best;
    return ORC_OK;
}

/* ------------------------------------------------------------------------------------------ */
/* Deterministic sampling                                                                       */
/* ------------------------------------------------------------------------------------------ */

/* PCG32 as [P4] "Deterministic sampling contract" freezes it: state' = state * 6364136223846793005 + inc
 * (mod 2^64); output = the 32-bit rotate-right of ((old >> 18) ^ old) >> 27 by old >> 59.  Seeding: state 0,
 * inc = 2 * stream_id + 1, advance, add the seed, advance. */
uint32_t orc_pcg32_next(orc_pcg32_t *r) {
    uint64_t old = r->state;
    r->state = old * 6364136223846793005ULL + r->inc;
    uint32_t xs = (uint32_t)(((old >> 18) ^ old) >> 27);
    uint32_t rot = (uint32_t)(old >> 59);
    return (xs >> rot) | (xs << ((32u - rot) & 31u));
}

void orc_pcg32_seed(uint64_t seed, uint64_t stream_id, orc_pcg32_t *r) {
    r->state = 0;
    r->inc = (stream_id << 1) | 1u;
    (void)orc_pcg32_next(r);
    r->state += seed;
    (void)orc_pcg32_next(r);
}

/* The high 24 bits of a word as a uniform in [0, 1): (r >> 8) * 2^-24, exact in f32 ([P4]). */
float orc_pcg32_uniform(uint32_t word) { return (float)(word >> 8) * (1.0f / 16777216.0f); }

typedef struct {
    float v;
    int32_t id;
} orc_cand_t;

/* descending value, ascending token id on equal values ([P1] section 7 "Tie-Breaking Sort") */
static int cand_cmp(const void *a, const void *b) {
    const orc_cand_t *x = (const orc_cand_t *)a, *y = (const orc_cand_t *)b;
    if (x->v > y->v) return -1;
    if (x->v < y->v) return 1;
    return x->id < y->id ? -1 : (x->id > y->id ? 1 : 0);
}

/* Steps 1-5 of the sampling order below, into z (vocab floats); seen: vocab zeroed bytes of scratch.  A +inf
 * value after them is a numerical failure. */
int32_t orc_sample_prepare(const float *logits, int32_t vocab, float penalty, const int32_t *history,
                           int32_t n_history, const int32_t *forbid, int32_t n_forbid, float *z, unsigned char *seen) {
    for (int32_t i = 0; i < vocab; ++i) z[i] = logits[i];
    for (int32_t j = 0; j < n_forbid; ++j)
        if (forbid[j] >= 0 && forbid[j] < vocab) z[forbid[j]] = -INFINITY;
    for (int32_t j = 0; j < n_history; ++j) {
        int32_t t = history[j];
        if (t < 0 || t >= vocab || seen[t]) continue;
        seen[t] = 1;
        if (z[t] > 0.0f) z[t] = z[t] / penalty;
        else if (z[t] < 0.0f) z[t] = z[t] * penalty;
    }
    for (int32_t i = 0; i < vocab; ++i) {
        if (isnan(z[i])) z[i] = -INFINITY;
        if (z[i] == 0.0f) z[i] = 0.0f;
        if (isinf(z[i]) && z[i] > 0.0f) return ORC_NUMERICAL_FAILURE;
    }
    return ORC_OK;
}

/* One token from a logits vector, following [P4] "Sampling order" (with [P1] section 7):
 *  1. copy the logits in token order; 2. forbidden tokens -> -inf; 3. repetition penalty on every token
 *  present in the history (counted once): a positive logit is divided by the penalty, a negative one
 *  multiplied; 4. NaN -> -inf; 5. -0 -> +0; a +inf logit is a numerical failure ([P1] section 4);
 *  6. temperature 0: the greatest logit, lowest id on ties, and no draw;
 *  7. otherwise divide by the temperature; 8. top-k by (value desc, id asc) among the finite logits;
 *  9. stable probabilities over the survivors (max subtracted, exp, sum in order, divide);
 *  10. order by (probability desc, id asc); 11. top-p: the shortest prefix whose cumulative probability is
 *  at least p (at least one token); 12. re-normalise the prefix ([P1] section 7); 13. draw u from the
 *  generator and take the first token whose cumulative probability exceeds u (the last one if rounding
 *  leaves every cumulative value at or below u).
 * Optional outputs: the final candidates' ids and probabilities in draw order, and their count. */
int32_t orc_sample(const float *logits, int32_t vocab, const orc_sample_params_t *p, const int32_t *history,
                   int32_t n_history, const int32_t *forbid, int32_t n_forbid, orc_pcg32_t *rng, int32_t *token,
                   float *probs_out, int32_t *ids_out, int32_t *n_out) {
    if (!logits || vocab <= 0 || !p || !token || n_history < 0 || n_forbid < 0) return ORC_INVALID_ARGUMENT;
    if (!(p->repetition_penalty > 0.0f) || isinf(p->repetition_penalty)) return ORC_INVALID_ARGUMENT;
    if (!(p->temperature >= 0.0f) || isinf(p->temperature)) return ORC_INVALID_ARGUMENT;
    if (p->temperature > 0.0f && (p->top_k < 1 || !(p->top_p > 0.0f) || !(p->top_p <= 1.0f) || !rng))
        return ORC_INVALID_ARGUMENT;
    float *z = (float *)malloc(sizeof(float) * (size_t)vocab);
    unsigned char *seen = (unsigned char *)calloc((size_t)vocab, 1);
    orc_cand_t *c = (orc_cand_t *)malloc(sizeof(orc_cand_t) * (size_t)vocab);
    float *pr = (float *)malloc(sizeof(float) * (size_t)vocab);
    int32_t rc = ORC_OK;
    if (!z || !seen || !c || !pr) {
        rc = ORC_INVALID_ARGUMENT;
        goto done;
    }
    rc = orc_sample_prepare(logits, vocab, p->repetition_penalty, history, n_history, forbid, n_forbid, z, seen);
    if (rc != ORC_OK) goto done;
    if (p->temperature == 0.0f) {
        int32_t best = -1;
        for (int32_t i = 0; i < vocab; ++i)
            if (z[i] > -INFINITY && (best < 0 || z[i] > z[best])) best = i;
        if (best < 0) {
            rc = ORC_NUMERICAL_FAILURE;
            goto done;
        }
        *token = best;
        if (ids_out) ids_out[0] = best;
        if (probs_out) probs_out[0] = 1.0f;
        if (n_out) *n_out = 1;
        goto done;
    }
    int32_t n = 0;
    for (int32_t i = 0; i < vocab; ++i) {
        float v = z[i] / p->temperature;
        if (isinf(v) && v > 0.0f) { /* a finite logit overflowed by the temperature division */
            rc = ORC_NUMERICAL_FAILURE;
            goto done;
        }
        if (v > -INFINITY) {
            c[n].v = v;
            c[n].id = i;
            ++n;
        }
    }
    if (n == 0) {
        rc = ORC_NUMERICAL_FAILURE;
        goto done;
    }
    qsort(c, (size_t)n, sizeof(orc_cand_t), cand_cmp);
    if (n > p->top_k) n = p->top_k;
    {
        const float m = c[0].v;
        float sum = 0.0f;
        for (int32_t j = 0; j < n; ++j) {
            pr[j] = orc_exp(c[j].v - m);
            sum = sum + pr[j];
        }
        for (int32_t j = 0; j < n; ++j) c[j].v = pr[j] / sum;
    }
    qsort(c, (size_t)n, sizeof(orc_cand_t), cand_cmp); /* (probability desc, id asc) */
    int32_t keep = n;
    {
        float cum = 0.0f;
        for (int32_t j = 0; j < n; ++j) {
            cum = cum + c[j].v;
            if (cum >= p->top_p) {
                keep = j + 1;
                break;
            }
        }
    }
    {
        float s2 = 0.0f;
        for (int32_t j = 0; j < keep; ++j) s2 = s2 + c[j].v;
        for (int32_t j = 0; j < keep; ++j) c[j].v = c[j].v / s2;
    }
    {
        const float u = orc_pcg32_uniform(orc_pcg32_next(rng));
        float cum = 0.0f;
        int32_t pick = keep - 1;
        for (int32_t j = 0; j < keep; ++j) {
            cum = cum + c[j].v;
            if (cum > u) {
                pick = j;
                break;
            }
        }
        *token = c[pick].id;
    }
    for (int32_t j = 0; j < keep; ++j) {
        if (ids_out) ids_out[j] = c[j].id;
        if (probs_out) probs_out[j] = c[j].v;
    }
    if (n_out) *n_out = keep;
done:
    free(z);
    free(seen);
    free(c);
    free(pr);
    return rc;
}

void orc_set_threads(int32_t n) {
    if (n > 0) omp_set_num_threads(n);
}
int32_t orc_get_threads(void) { return omp_get_max_threads(); }

/* ------------------------------------------------------------------------------------------ */
/* Whole model                                                                                  */
/* ------------------------------------------------------------------------------------------ */

struct orc_model {
    orc_cfg_t c;
    orc_mat_t embed;
    const void *final_norm;
    orc_layer_t *layers;
    float *k_cache, *v_cache; /* [seq][layer][kv_head][pos][head_dim] */
    int32_t *len;
};

/* KV layout [Layer][Head][Position][Dim] per sequence ([P1] section 6 "Layout and Ownership"). */
static size_t kv_index(const orc_model_t *m, int32_t seq, int32_t layer, int32_t head, int32_t pos) {
    const orc_cfg_t *c = &m->c;
    return ((((size_t)seq * c->n_layers + layer) * c->n_kv_heads + head) * (size_t)c->max_ctx + pos) *
           (size_t)c->head_dim;
}

orc_model_t *orc_create(const orc_cfg_t *cfg, const orc_mat_t *embed, const void *final_norm,
                        const orc_layer_t *layers) {
    if (!cfg || cfg->n_q_heads <= 0 || cfg->n_kv_heads <= 0 || cfg->n_q_heads % cfg->n_kv_heads) return NULL;
    if (cfg->head_dim % 2 || cfg->max_ctx <= 0 || cfg->n_seq <= 0) return NULL;
    if (cfg->fmt < ORC_FMT_BF16 || cfg->fmt > ORC_FMT_Q8_ACT8) return NULL;
    /* quantized blocks of 32 along every contraction: no tail groups ([P1] section 3, a shape failing the
     * modulo-32 check is an initialisation fault) */
    if (cfg->fmt != ORC_FMT_BF16 &&
        (cfg->hidden % 32 || (cfg->n_q_heads * cfg->head_dim) % 32 || cfg->inter % 32))
        return NULL;
    orc_model_t *m = (orc_model_t *)calloc(1, sizeof(orc_model_t));
    if (!m) return NULL;
    m->c = *cfg;
    if (embed) m->embed = *embed;
    m->final_norm = final_norm;
    m->layers = (orc_layer_t *)malloc(sizeof(orc_layer_t) * (size_t)cfg->n_layers);
    memcpy(m->layers, layers, sizeof(orc_layer_t) * (size_t)cfg->n_layers);
    size_t kv = (size_t)cfg->n_seq * cfg->n_layers * cfg->n_kv_heads * (size_t)cfg->max_ctx * cfg->head_dim;
    m->k_cache = (float *)calloc(kv, sizeof(float));
    m->v_cache = (float *)calloc(kv, sizeof(float));
    m->len = (int32_t *)calloc((size_t)cfg->n_seq, sizeof(int32_t));
    if (!m->layers || !m->k_cache || !m->v_cache || !m->len) {
        orc_destroy(m);
        return NULL;
    }
    return m;
}

void orc_destroy(orc_model_t *m) {
    if (!m) return;
    free(m->layers);
    free(m->k_cache);
    free(m->v_cache);
    free(m->len);
    free(m);
}

int32_t orc_set_len(orc_model_t *m, int32_t seq, int32_t len) {
    if (seq < 0 || seq >= m->c.n_seq || len < 0 || len > m->c.max_ctx) return ORC_INVALID_ARGUMENT;
    m->len[seq] = len;
    return ORC_OK;
}

int32_t orc_get_len(const orc_model_t *m, int32_t seq) { return (seq < 0 || seq >= m->c.n_seq) ? -1 : m->len[seq]; }

/* k, v: [n_kv_heads][n_pos][head_dim] bf16 bits. */
int32_t orc_kv_write(orc_model_t *m, int32_t seq, int32_t layer, int32_t pos0, int32_t n_pos, const uint16_t *k,
                     const uint16_t *v) {
    const orc_cfg_t *c = &m->c;
    if (seq < 0 || seq >= c->n_seq || layer < 0 || layer >= c->n_layers || pos0 < 0 || n_pos < 0 ||
        pos0 + n_pos > c->max_ctx)
        return ORC_INVALID_ARGUMENT;
    for (int32_t h = 0; h < c->n_kv_heads; ++h)
        for (int32_t p = 0; p < n_pos; ++p) {
            size_t dst = kv_index(m, seq, layer, h, pos0 + p);
            size_t src = ((size_t)h * n_pos + p) * c->head_dim;
            for (int32_t d = 0; d < c->head_dim; ++d) {
                m->k_cache[dst + d] = orc_bf16_to_f32(k[src + d]);
                m->v_cache[dst + d] = orc_bf16_to_f32(v[src + d]);
            }
        }
    return ORC_OK;
}

int32_t orc_kv_read(const orc_model_t *m, int32_t seq, int32_t layer, int32_t pos0, int32_t n_pos, uint16_t *k,
                    uint16_t *v) {
    const orc_cfg_t *c = &m->c;
    if (seq < 0 || seq >= c->n_seq || layer < 0 || layer >= c->n_layers || pos0 < 0 || n_pos < 0 ||
        pos0 + n_pos > c->max_ctx)
        return ORC_INVALID_ARGUMENT;
    for (int32_t h = 0; h < c->n_kv_heads; ++h)
        for (int32_t p = 0; p < n_pos; ++p) {
            size_t src = kv_index(m, seq, layer, h, pos0 + p);
            size_t dst = ((size_t)h * n_pos + p) * c->head_dim;
            for (int32_t d = 0; d < c->head_dim; ++d) {
                k[dst + d] = orc_f32_to_bf16(m->k_cache[src + d]);
                v[dst + d] = orc_f32_to_bf16(m->v_cache[src + d]);
            }
        }
    return ORC_OK;
}

static void load_norm(const void *w, int32_t fmt, int32_t n, float *out) {
    for (int32_t i = 0; i < n; ++i) out[i] = norm_weight(w, fmt, i);
}

/* One decoder layer for one token at position pos, following the step order of [P1] section 5
 * "Transformer Layer Execution Loop" (and section 2 items 1-6). x is updated in place. */
/* A layer projection: q8 x q8 with dynamically quantized activations in the Q8_ACT8 format, else the f32
 * activation dot of the weight format. */
static void layer_matvec(const orc_cfg_t *c, const orc_mat_t *m, const float *x, float *out) {
    if (c->fmt == ORC_FMT_Q8_ACT8) matvec_act8(m, x, out);
    else orc_matvec(m, x, out);
}

/* force / own: NULL, or this layer's [2][HKV][D] bf16 bits (K heads, then V heads) of the appended position:
 * `own` receives the oracle's own rounded values, `force` replaces them in the cache (teacher forcing of the
 * current position; the caller checks that the two differ by rounding only). */
static int32_t decode_layer(orc_model_t *m, int32_t seq, int32_t l, int32_t pos, float *x, const uint16_t *force,
                            uint16_t *own) {
    const orc_cfg_t *c = &m->c;
    const orc_layer_t *W = &m->layers[l];
    const int32_t H = c->hidden, D = c->head_dim, HQ = c->n_q_heads, HKV = c->n_kv_heads;
    float *residual = (float *)malloc(sizeof(float) * H);
    float *xn = (float *)malloc(sizeof(float) * (size_t)(H > c->inter ? H : c->inter));
    float *w = (float *)malloc(sizeof(float) * (size_t)H);
    float *q = (float *)malloc(sizeof(float) * (size_t)HQ * D);
    float *k = (float *)malloc(sizeof(float) * (size_t)HKV * D);
    float *v = (float *)malloc(sizeof(float) * (size_t)HKV * D);
    float *attn = (float *)malloc(sizeof(float) * (size_t)HQ * D);
    float *gate = (float *)malloc(sizeof(float) * (size_t)c->inter);
    float *up = (float *)malloc(sizeof(float) * (size_t)c->inter);
    float *act = (float *)malloc(sizeof(float) * (size_t)c->inter);
    float *proj = (float *)malloc(sizeof(float) * (size_t)H);
    float *cs = (float *)malloc(sizeof(float) * (size_t)D);
    int32_t rc = ORC_OK;

    memcpy(residual, x, sizeof(float) * H);

    /* 1. pre-attention RMSNorm */
    load_norm(W->attn_norm, c->fmt, H, w);
    orc_rmsnorm(x, w, H, c->eps, xn);

    /* 2. Q, K, V projections (no bias) */
    layer_matvec(c, &W->q, xn, q);
    layer_matvec(c, &W->k, xn, k);
    layer_matvec(c, &W->v, xn, v);

    /* 3. QK-Norm: RMSNorm over each head_dim slice, one shared weight per projection */
    float *hw = w; /* reuse: head_dim <= hidden */
    float *tmp = proj;
    load_norm(W->q_norm, c->fmt, D, hw);
    for (int32_t h = 0; h < HQ; ++h) {
        orc_rmsnorm(q + (size_t)h * D, hw, D, c->eps, tmp);
        memcpy(q + (size_t)h * D, tmp, sizeof(float) * D);
    }
    load_norm(W->k_norm, c->fmt, D, hw);
    for (int32_t h = 0; h < HKV; ++h) {
        orc_rmsnorm(k + (size_t)h * D, hw, D, c->eps, tmp);
        memcpy(k + (size_t)h * D, tmp, sizeof(float) * D);
    }

    /* 4. RoPE on the normalised queries and keys */
    float *cos_t = cs, *sin_t = cs + D / 2;
    orc_rope_table(c->theta, D, pos, cos_t, sin_t);
    for (int32_t h = 0; h < HQ; ++h) orc_rope_apply(q + (size_t)h * D, D, cos_t, sin_t);
    for (int32_t h = 0; h < HKV; ++h) orc_rope_apply(k + (size_t)h * D, D, cos_t, sin_t);

    /* 5. KV append at [seq][layer][head][pos]; the cache element type is bf16 (rounded to nearest
     *    even), unless the model was created with f32 KV */
    for (int32_t h = 0; h < HKV; ++h)
        for (int32_t d = 0; d < D; ++d) {
            size_t at = kv_index(m, seq, l, h, pos) + d;
            float kf = k[(size_t)h * D + d], vf = v[(size_t)h * D + d];
            const size_t ki = (size_t)h * D + d, vi = (size_t)HKV * D + ki;
            if (own) {
                own[ki] = orc_f32_to_bf16(kf);
                own[vi] = orc_f32_to_bf16(vf);
            }
            if (force) {
                m->k_cache[at] = orc_bf16_to_f32(force[ki]);
                m->v_cache[at] = orc_bf16_to_f32(force[vi]);
            } else {
                m->k_cache[at] = c->kv_f32 ? kf : orc_bf16_to_f32(orc_f32_to_bf16(kf));
                m->v_cache[at] = c->kv_f32 ? vf : orc_bf16_to_f32(orc_f32_to_bf16(vf));
            }
        }

    /* 6. grouped-query attention over positions 0..pos of this layer's cache */
    {
        size_t head_stride = (size_t)c->max_ctx * D;
        size_t base = kv_index(m, seq, l, 0, 0);
        rc = orc_gqa_attention(q, HQ, HKV, m->k_cache + base, m->v_cache + base, head_stride, pos + 1, D, attn);
    }
    if (rc != ORC_OK) goto done;

    /* 7. output projection and residual */
    layer_matvec(c, &W->o, attn, proj);
    for (int32_t i = 0; i < H; ++i) x[i] = residual[i] + proj[i];
    memcpy(residual, x, sizeof(float) * H);

    /* 8. post-attention RMSNorm, SwiGLU MLP, residual */
    load_norm(W->mlp_norm, c->fmt, H, w);
    orc_rmsnorm(x, w, H, c->eps, xn);
    layer_matvec(c, &W->gate, xn, gate);
    layer_matvec(c, &W->up, xn, up);
    for (int32_t i = 0; i < c->inter; ++i) {
        float sig = 1.0f / (1.0f + orc_exp(-gate[i]));
        act[i] = (gate[i] * sig) * up[i];
    }
    layer_matvec(c, &W->down, act, proj);
    for (int32_t i = 0; i < H; ++i) x[i] = residual[i] + proj[i];

done:
    free(residual);
    free(xn);
    free(w);
    free(q);
    free(k);
    free(v);
    free(attn);
    free(gate);
    free(up);
    free(act);
    free(proj);
    free(cs);
    return rc;
}

int32_t orc_step(orc_model_t *m, int32_t seq, int32_t tok, const float *hidden_in, float *hidden_out,
                 float *logits, int32_t *argmax) {
    return orc_step_kv(m, seq, tok, hidden_in, hidden_out, logits, argmax, NULL, NULL);
}

/* orc_step with the appended position's bf16 K/V taken from kv_force ([L][2][HKV][D] bits) instead of the
 * oracle's own rounding, which is written to kv_own (same layout) when given.  Only for a bf16 cache. */
int32_t orc_step_kv(orc_model_t *m, int32_t seq, int32_t tok, const float *hidden_in, float *hidden_out,
                    float *logits, int32_t *argmax, const uint16_t *kv_force, uint16_t *kv_own) {
    const orc_cfg_t *c = &m->c;
    if (seq < 0 || seq >= c->n_seq) return ORC_INVALID_ARGUMENT;
    if (kv_force && c->kv_f32) return ORC_INVALID_ARGUMENT;
    const size_t per_layer = (size_t)2 * c->n_kv_heads * c->head_dim;
    if (c->n_q_heads > 1024) return ORC_UNSUPPORTED_SHAPE;
    int32_t pos = m->len[seq];
    /* a position at or past the admitted context is a typed error; no ring buffering
     * ([P1] section 6 "Maximum Context Overflow") */
    if (pos >= c->max_ctx) return ORC_CONTEXT_EXCEEDED;
    const int32_t H = c->hidden;
    float *x = (float *)malloc(sizeof(float) * H);
    int32_t rc = ORC_OK;
    if (c->input_mode == 1) {
        if (!hidden_in) {
            free(x);
            return ORC_INVALID_ARGUMENT;
        }
        memcpy(x, hidden_in, sizeof(float) * H);
    } else {
        /* embedding: row `tok` of the tied table ([P1] section 2, initial hidden state) */
        if (tok < 0 || tok >= c->vocab) {
            free(x);
            return ORC_INVALID_ARGUMENT;
        }
        orc_dequant_row(&m->embed, tok, x);
    }
    for (int32_t l = 0; l < c->n_layers && rc == ORC_OK; ++l)
        rc = decode_layer(m, seq, l, pos, x, kv_force ? kv_force + (size_t)l * per_layer : NULL,
                          kv_own ? kv_own + (size_t)l * per_layer : NULL);
    if (rc == ORC_OK && hidden_out) {
        for (int32_t i = 0; i < H; ++i)
            if (!isfinite(x[i])) rc = ORC_NUMERICAL_FAILURE;
        memcpy(hidden_out, x, sizeof(float) * H);
    }
    if (rc == ORC_OK && c->input_mode == 0 && (logits || argmax)) {
        /* final RMSNorm and tied logits: logits_t = sum_i E_ti * xn_i ([P1] section 2 item 7) */
        float *w = (float *)malloc(sizeof(float) * H);
        float *xn = (float *)malloc(sizeof(float) * H);
        float *lg = logits ? logits : (float *)malloc(sizeof(float) * (size_t)c->vocab);
        load_norm(m->final_norm, c->fmt, H, w);
        orc_rmsnorm(x, w, H, c->eps, xn);
        orc_matvec(&m->embed, xn, lg);
        int32_t best = 0;
        rc = orc_argmax(lg, c->vocab, &best);
        if (argmax) *argmax = best;
        if (!logits) free(lg);
        free(w);
        free(xn);
    }
    free(x);
    /* commit: the appended position becomes valid only after the whole step succeeded
     * ([P4] "Cancellation", partially written positions stay invalid) */
    if (rc == ORC_OK) m->len[seq] = pos + 1;
    return rc;
}
