/*
 * Seeded synthetic input generator.
 *
 * Test and benchmark infrastructure shared by both sides of the parity check:
 * it only draws random numbers and rounds them to storage types.  It holds
 * none of the decoder's arithmetic.
 *
 * Random words come from PCG32 as defined on "Portable WebAssembly Runtime
 * Architecture for TinyRustLM", section "Threads, Scheduling, Cache Identity,
 * and Deterministic Sampling" (transition, output permutation, seeding by
 * stream id and seed, and the 24-bit uniform conversion).
 *
 * Every tensor is cut into chunks of SYN_CHUNK elements; chunk c of tensor t
 * draws from its own PCG32 stream (t << 32 | c), so the output does not
 * depend on how many threads generate it.
 *
 * Normals: Box-Muller on two uniforms u1, u2 in [0,1): r = sqrt(-2 ln(1-u1)),
 * z0 = r cos(2 pi u2), z1 = r sin(2 pi u2), evaluated in double.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define SYN_CHUNK 65536ULL

typedef struct {
    uint64_t state;
    uint64_t inc;
} pcg32_t;

static uint32_t pcg32_next(pcg32_t *g) {
    uint64_t old = g->state;
    g->state = old * 6364136223846793005ULL + g->inc;
    uint32_t xorshifted = (uint32_t)(((old >> 18) ^ old) >> 27);
    uint32_t rot = (uint32_t)(old >> 59);
    return (xorshifted >> rot) | (xorshifted << ((32u - rot) & 31u));
}

static void pcg32_seed(pcg32_t *g, uint64_t seed, uint64_t stream_id) {
    g->state = 0;
    g->inc = (stream_id << 1) | 1u;
    (void)pcg32_next(g);
    g->state += seed;
    (void)pcg32_next(g);
}

static double u24(pcg32_t *g) { return (double)(pcg32_next(g) >> 8) * (1.0 / 16777216.0); }

static uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (uint16_t)((u >> 16) | 0x40u);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7fffu + lsb;
    return (uint16_t)(u >> 16);
}

uint32_t syn_pcg32_words(uint64_t seed, uint64_t stream_id, uint64_t n, uint32_t *out) {
    pcg32_t g;
    pcg32_seed(&g, seed, stream_id);
    for (uint64_t i = 0; i < n; ++i) out[i] = pcg32_next(&g);
    return 0;
}

/* Fills n values; kind selects what one element is. */
enum { SYN_NORMAL_F32 = 0, SYN_NORMAL_BF16 = 1, SYN_UNIFORM_F32 = 2, SYN_INT8 = 3, SYN_INT32 = 4 };

static void fill_chunk(int kind, uint64_t seed, uint64_t tensor_id, uint64_t c, uint64_t n0, uint64_t n1, double a,
                       double b, void *out) {
    pcg32_t g;
    pcg32_seed(&g, seed, (tensor_id << 32) | c);
    if (kind == SYN_NORMAL_F32 || kind == SYN_NORMAL_BF16) {
        for (uint64_t i = n0; i < n1; i += 2) {
            double u1 = u24(&g), u2 = u24(&g);
            double r = sqrt(-2.0 * log(1.0 - u1));
            double z[2] = {r * cos(2.0 * M_PI * u2), r * sin(2.0 * M_PI * u2)};
            for (int k = 0; k < 2 && i + k < n1; ++k) {
                float f = (float)(a + b * z[k]);
                if (kind == SYN_NORMAL_F32)
                    ((float *)out)[i + k] = f;
                else
                    ((uint16_t *)out)[i + k] = f32_to_bf16_rne(f);
            }
        }
    } else if (kind == SYN_UNIFORM_F32) {
        for (uint64_t i = n0; i < n1; ++i) ((float *)out)[i] = (float)(a + (b - a) * u24(&g));
    } else {
        /* uniform integer in [a, b] by rejection on 32-bit words */
        int64_t lo = (int64_t)a, hi = (int64_t)b;
        uint64_t range = (uint64_t)(hi - lo + 1);
        uint64_t limit = (1ULL << 32) - ((1ULL << 32) % range);
        for (uint64_t i = n0; i < n1; ++i) {
            uint32_t r;
            do r = pcg32_next(&g);
            while ((uint64_t)r >= limit);
            int64_t v = lo + (int64_t)((uint64_t)r % range);
            if (kind == SYN_INT8)
                ((int8_t *)out)[i] = (int8_t)v;
            else
                ((int32_t *)out)[i] = (int32_t)v;
        }
    }
}

/* kind: see enum; for normals a=mean b=std; uniform a=lo b=hi; ints a=lo b=hi (inclusive). */
uint32_t syn_fill(int kind, uint64_t seed, uint64_t tensor_id, uint64_t n, double a, double b, void *out) {
    if (kind < 0 || kind > SYN_INT32) return 1;
    uint64_t nchunks = (n + SYN_CHUNK - 1) / SYN_CHUNK;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t c = 0; c < (int64_t)nchunks; ++c) {
        uint64_t n0 = (uint64_t)c * SYN_CHUNK;
        uint64_t n1 = n0 + SYN_CHUNK < n ? n0 + SYN_CHUNK : n;
        fill_chunk(kind, seed, tensor_id, (uint64_t)c, n0, n1, a, b, out);
    }
    return 0;
}
