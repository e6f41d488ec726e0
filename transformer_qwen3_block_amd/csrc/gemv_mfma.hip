// Batched Q8 matrix-vector products for a decode step of 2..16 sequences on gfx950 MFMA.
//
// y[s][row] = sum_k x[s][k] * (q[row][k] * scale[row][k/32]) for every sequence s < S: the weights stream from
// HBM once for all sequences.  One v_mfma_f32_16x16x32_f16 covers 16 sequences x 16 weight rows x one
// 32-column Q8 block.  The int8 codes are exact in f16; each activation is split into an f16 high part and
// an f16 remainder (x = hi + lo to about 22 significant bits); both products accumulate in f32, and the
// block's f32 scale multiplies the block's partial sum -- the per-block factoring of the dequantised dot
// product of [P1] section 5, a reassociation of the same sum.
//
// Lane layout of v_mfma_f32_16x16x32_f16 (wave64): lane l supplies A[l%16][8*(l/16)+e] (sequence l%16, block
// column 8*(l/16)+e) and B[8*(l/16)+e][l%16] (weight row l%16 of the tile), and receives C[4*(l/16)+r][l%16]
// (sequence 4*(l/16)+r, row l%16).
//
// A workgroup of KW waves splits K: wave w owns blocks [w*NB, (w+1)*NB), forms its activation operands once
// (RMSNorm inputs from the f32 residual stream and the per-tile sums of squares the residual epilogues leave;
// attention outputs and SwiGLU activations as the f16 pairs their producers wrote) and keeps them in
// registers for every 16-row tile it visits (grid-stride over tiles, the next tile's
// codes in flight while the current one is multiplied); the waves' partial tiles are summed in LDS in wave
// order, so every output element has a fixed summation order.  Epilogues: store (Q/K/V), residual add (o_proj,
// down; also the per-tile sums of squares of the updated rows, which the next RMSNorm reads in tile order),
// SwiGLU (gate/up rows interleaved in the tile so gate and up of a unit meet in one 16-lane row) and logits
// with per-workgroup greedy partials.
//
// Page titles used in citations:
//   [P1] "Scalar-Native Qwen3 Reference Runtime As The Numerical Authority"
//   [P4] "Portable WebAssembly Runtime Architecture for TinyRustLM"
#include <math.h>

#include "common.h"

namespace qw3 {

namespace {

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma16(const uint4 &a, const uint4 &b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                  0, 0, 0);
}

// Eight int8 codes -> eight f16 (exact: |q| <= 127).
__device__ __forceinline__ uint4 codes_to_f16(uint2 w) {
    f16x8_t h;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        h[e] = (_Float16)(int)(int8_t)(w.x >> (8 * e));
        h[4 + e] = (_Float16)(int)(int8_t)(w.y >> (8 * e));
    }
    return __builtin_bit_cast(uint4, h);
}

// Component-wise select of two 16-byte values.  (A conditional expression on the struct type can make the
// compiler select between two addresses and keep the operands in scratch memory.)
__device__ __forceinline__ uint4 sel4(bool c, const uint4 &a, const uint4 &b) {
    return make_uint4(c ? a.x : b.x, c ? a.y : b.y, c ? a.z : b.z, c ? a.w : b.w);
}
// 16-byte load through the vector type (stays in registers)
__device__ __forceinline__ uint4 ld16(const void *p) {
    const u32x4_t v = *(const u32x4_t *)p;
    return make_uint4(v.x, v.y, v.z, v.w);
}

// max that keeps a NaN: once either operand is NaN the result is NaN (fmaxf would drop it)
__device__ __forceinline__ float nan_max(float a, float b) { return (b > a || b != b) ? b : a; }

// f32 -> (f16 high part, f16 remainder) bits
__device__ __forceinline__ void split_one(float v, uint16_t &hi, uint16_t &lo) {
    const _Float16 h = (_Float16)v;
    hi = __builtin_bit_cast(uint16_t, h);
    lo = __builtin_bit_cast(uint16_t, (_Float16)(v - (float)h));
}

// A8 (the q8 x q8 weight format): the activations are quantized to int8 per (sequence, 32-column block) while the
// wave forms its operands ([P3] section 5 "Q8_0 Mixed-Precision Matrix Multiplication": block scale max|x| / 127,
// codes rounded to nearest with ties away from zero, clamped to [-127, 127]) and each block is one
// v_mfma_i32_16x16x32_i8 (lane l: A = sequence l%16, B = weight row l%16, columns 8*(l/16)..+8 of the block),
// whose int32 sums are scaled by both block scales, (float)isum * (weight scale * activation scale), and
// added block by block.  The inputs are the f32 values: the residual stream through the RMSNorm, or the f32
// outputs of the attention and SwiGLU.
template <int KW, int NB, int EPI, bool A8 = false>
__global__ __launch_bounds__(64 * KW) void gemv_mfma_kernel(GemvArgs a) {
    static_assert(NB % 2 == 0, "blocks come in pairs");
    constexpr int NP = NB / 2;        // 64-column block pairs per wave
    __shared__ float red[KW][4][64];  // per wave: C[4*(l/16)+r][l%16] of lane l at [r][l]
    __shared__ float s_inv[kMaxSeq];
    __shared__ __attribute__((aligned(16))) float s_gw[EPI == EPI_RESID ? 1 : KW][NB * 32];  // norm weight slices
    __shared__ __attribute__((aligned(16))) float s_da[A8 ? KW : 1][A8 ? NB : 1][kMaxSeq];  // A8: activation scales

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q = lane >> 4, c = lane & 15;  // column group, sequence (A) / row slot (B, C)
    const bool first = q < 2;                // groups 0, 1 hold the pair's first block, 2, 3 its second
    const int S = a.S, K = a.K, KB = K / 32;
    const int kb0 = w * NB;
    const int8_t *wq = (const int8_t *)a.w;

    // weight row of row slot c in tile t (SwiGLU tiles: rows 0-7 gate units, 8-15 the matching up units)
    auto wrow = [&](int t) -> long long {
        if constexpr (EPI == EPI_SWIGLU) {
            const int unit = t * 8 + (c & 7);
            return c < 8 ? (long long)unit : (long long)a.N + unit;
        } else {
            return (long long)min(t * 16 + c, a.N - 1);
        }
    };
    const int ntiles = EPI == EPI_SWIGLU ? a.N / 8 : (a.N + 15) / 16;
    // Lane (q, c) reads 16 codes of row c: columns 16q..16q+15 of each 64-column block pair (one 16-byte
    // load; four lanes cover 64 contiguous bytes of a row), and the row's scales of this wave's blocks.
    auto load_tile = [&](int t, uint4 (&cw)[NP], float (&sc)[NB]) {
        const long long row = wrow(t < ntiles ? t : 0);
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const u32x4_t v = __builtin_nontemporal_load((const u32x4_t *)(wq + row * K + (kb0 + 2 * p) * 32 + 16 * q));
            cw[p] = make_uint4(v.x, v.y, v.z, v.w);
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) sc[j] = a.scales[row * KB + kb0 + j];
    };

    // This wave's activations go out first, then the first tile's codes (and the sums of squares): one memory
    // round trip before the first product, the activations converted while the codes still stream (loads
    // return in order).  Activation operands: lane (q, c) holds sequence c's columns
    // 16q..16q+15 of each block pair, as f16 high parts and remainders (a1: first eight, a2: last eight).
    uint4 cw[NP];
    float sc[NB];
    int t = blockIdx.x;
    const uint4 z4 = make_uint4(0, 0, 0, 0);
    constexpr int kSsqPer = 1024 / 16 / 16;  // RMSNorm inputs have K = 1024: 64 tile sums, 4 per thread
    uint4 a1h[NP], a1l[NP], a2h[NP], a2l[NP];  // f16 operands (high part, remainder)
    uint2 cw8[NB], ac[NB];  // A8: the tile's weight codes and the activation codes, columns 8q..8q+7 of each block
    auto load_tile8 = [&](int t, uint2 (&cw)[NB], float (&sc)[NB]) {
        const long long row = wrow(t < ntiles ? t : 0);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const u32x2_t v = __builtin_nontemporal_load((const u32x2_t *)(wq + row * K + (kb0 + b) * 32 + 8 * q));
            cw[b] = make_uint2(v.x, v.y);
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) sc[j] = a.scales[row * KB + kb0 + j];
    };
    if constexpr (!A8) {
        if (EPI != EPI_RESID && a.norm_w) {
            // RMSNorm input ([P1] section 2 items 1 and 6): w * (x * inv) with inv = 1 / sqrt(mean(x^2) + eps) of
            // the sequence, from the per-16-row sums of squares (tile order, then a fixed 16-lane tree); the
            // residual stream itself may exceed the f16 range, the normalised operand does not
            // the tile sums of squares go out first: waiting for them does not wait for the later loads
            float ssv[kSsqPer];
            const int ss_s = tid >> 4, ss_p = tid & 15;
    #pragma unroll
            for (int i = 0; i < kSsqPer; ++i)  // unconditional (in bounds for every thread); absent ones unused
                ssv[i] = a.ssq[(ss_p + 16 * i) * kMaxSeq + (ss_s & (kMaxSeq - 1))];
            asm volatile("" ::: "memory");  // keep these loads ahead of the others (loads return in order)
            // the wave's slice of the norm weight (NB * 32 = 256 floats) is read once, into LDS, instead of by
            // each of the 16 sequence lanes
            static_assert(EPI == EPI_RESID || NB * 32 == 4 * 64, "one 16-byte norm weight chunk per lane");
            const float4 gwl = *(const float4 *)(a.norm_w + kb0 * 32 + 4 * lane);
            float xv[NP][16], gv[NP][16];
            const int xrow = c < S ? c : S - 1;  // lanes of absent sequences read a present row (zeroed below)
    #pragma unroll
            for (int p = 0; p < NP; ++p) {
                const int k = (kb0 + 2 * p) * 32 + 16 * q;
    #pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float4 xx = *(const float4 *)(a.x + (size_t)xrow * a.ldx + k + 4 * i);
                    xv[p][4 * i] = xx.x; xv[p][4 * i + 1] = xx.y; xv[p][4 * i + 2] = xx.z; xv[p][4 * i + 3] = xx.w;
                }
            }
            load_tile(t, cw, sc);  // after the activations: they return first and are converted while codes stream
            *(float4 *)&s_gw[w][4 * lane] = gwl;
            if (tid < 256) {
                float ss = 0.f;
    #pragma unroll
                for (int i = 0; i < kSsqPer; ++i) ss += ss_s < S ? ssv[i] : 0.f;
                ss = row16_sum(ss);
                if (ss_p == 0) s_inv[ss_s] = 1.0f / sqrtf(ss / (float)K + a.eps);
            }
            __syncthreads();
            const float inv = s_inv[c];
    #pragma unroll
            for (int p = 0; p < NP; ++p)
    #pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float4 gg = *(const float4 *)&s_gw[w][2 * p * 32 + 16 * q + 4 * i];
                    gv[p][4 * i] = gg.x; gv[p][4 * i + 1] = gg.y; gv[p][4 * i + 2] = gg.z; gv[p][4 * i + 3] = gg.w;
                }
    #pragma unroll
            for (int p = 0; p < NP; ++p) {
                f16x8_t h1, l1, h2, l2;
    #pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float v1 = c < S ? gv[p][e] * (xv[p][e] * inv) : 0.f;
                    const float v2 = c < S ? gv[p][8 + e] * (xv[p][8 + e] * inv) : 0.f;
                    h1[e] = (_Float16)v1;
                    l1[e] = (_Float16)(v1 - (float)h1[e]);
                    h2[e] = (_Float16)v2;
                    l2[e] = (_Float16)(v2 - (float)h2[e]);
                }
                a1h[p] = __builtin_bit_cast(uint4, h1);
                a1l[p] = __builtin_bit_cast(uint4, l1);
                a2h[p] = __builtin_bit_cast(uint4, h2);
                a2l[p] = __builtin_bit_cast(uint4, l2);
            }
        } else {
            // operand written by the previous kernel (attention output, SwiGLU activations)
    #pragma unroll
            for (int p = 0; p < NP; ++p) {
                const size_t o = (((size_t)(kb0 / 2 + p) * 4 + q) * kMaxSeq + c) * 16;
                const bool on = c < S;  // absent sequences: zero operands, no read outside this batch's slots
                const size_t oc = on ? o : 0;  // absent sequences read slot 0 and are zeroed
                a1h[p] = sel4(on, ld16(a.a_hi + oc), z4);
                a2h[p] = sel4(on, ld16(a.a_hi + oc + 8), z4);
                a1l[p] = sel4(on, ld16(a.a_lo + oc), z4);
                a2l[p] = sel4(on, ld16(a.a_lo + oc + 8), z4);
            }
            load_tile(t, cw, sc);
        }
    } else {
        // f32 inputs of sequence c (lanes of absent sequences read a present row and take zeros), the tile's
        // codes behind them; then per block the 32 values of a sequence sit in the four lanes c, c+16, c+32,
        // c+48, which share the block's max through two shuffles
        constexpr bool kNorm = EPI != EPI_RESID;
        const bool norm = kNorm && a.norm_w;
        const bool on = c < S;
        const int xrow = on ? c : S - 1;
        float ssv[kSsqPer];
        const int ss_s = tid >> 4, ss_p = tid & 15;
        float4 gwl = make_float4(0.f, 0.f, 0.f, 0.f);
        if (norm) {
#pragma unroll
            for (int i = 0; i < kSsqPer; ++i)
                ssv[i] = a.ssq[(ss_p + 16 * i) * kMaxSeq + (ss_s & (kMaxSeq - 1))];
            gwl = *(const float4 *)(a.norm_w + kb0 * 32 + 4 * lane);
        }
        float xv[NB][8];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const float *xp = a.x + (size_t)xrow * a.ldx + (kb0 + b) * 32 + 8 * q;
            const float4 x0 = *(const float4 *)xp, x1 = *(const float4 *)(xp + 4);
            xv[b][0] = x0.x; xv[b][1] = x0.y; xv[b][2] = x0.z; xv[b][3] = x0.w;
            xv[b][4] = x1.x; xv[b][5] = x1.y; xv[b][6] = x1.z; xv[b][7] = x1.w;
        }
        load_tile8(t, cw8, sc);
        float inv = 1.f;
        if constexpr (kNorm) {
            if (norm) {
                *(float4 *)&s_gw[w][4 * lane] = gwl;
                if (tid < 256) {
                    float ss = 0.f;
#pragma unroll
                    for (int i = 0; i < kSsqPer; ++i) ss += ss_s < S ? ssv[i] : 0.f;
                    ss = row16_sum(ss);
                    if (ss_p == 0) s_inv[ss_s] = 1.0f / sqrtf(ss / (float)K + a.eps);
                }
                __syncthreads();
                inv = s_inv[c];
            }
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            float v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                v[e] = xv[b][e];
                if constexpr (kNorm)
                    if (norm) v[e] = s_gw[w][b * 32 + 8 * q + e] * (v[e] * inv);
                if (!on) v[e] = 0.f;
            }
            // block max of |v|, NaN-sticky (a NaN anywhere in the block makes it NaN)
            float m = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) m = nan_max(m, fabsf(v[e]));
            m = nan_max(m, __shfl_xor(m, 16, 64));
            m = nan_max(m, __shfl_xor(m, 32, 64));
            const float d = m / 127.0f;  // NaN stays NaN
            const bool ok = d > 0.f && d < INFINITY;
            uint32_t lo = 0, hi = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float c0 = ok ? fminf(fmaxf(roundf(v[e] / d), -127.f), 127.f) : 0.f;
                const float c1 = ok ? fminf(fmaxf(roundf(v[4 + e] / d), -127.f), 127.f) : 0.f;
                lo |= ((uint32_t)(int)c0 & 0xffu) << (8 * e);
                hi |= ((uint32_t)(int)c1 & 0xffu) << (8 * e);
            }
            ac[b] = make_uint2(lo, hi);
            if (q == 0) s_da[w][b][c] = d;
        }
        __syncthreads();  // every sequence's block scales, for the lanes that scale its outputs
    }

    // logits: running greedy choice of this thread's (sequence, row slot)
    float best = -INFINITY;
    int besti = 0x7fffffff, bad = 0;
    const int es = tid >> 4, er = tid & 15;  // epilogue thread: sequence, row slot

    // The residual products launch one workgroup per tile; the others walk several tiles with the next
    // tile's codes in flight.
    constexpr bool kStride = EPI != EPI_RESID;
    for (; t < ntiles; t += gridDim.x) {
        uint4 cn[NP];
        uint2 cn8[NB];
        float sn[NB];
        if constexpr (kStride) {
            if constexpr (A8)
                load_tile8(t + gridDim.x, cn8, sn);
            else
                load_tile(t + gridDim.x, cn, sn);
        }
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        if constexpr (A8) {
            // one int8 product per block: lane l's four outputs are sequences 4*(l/16)..+3 of weight row l%16
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const i32x4_t ci = __builtin_amdgcn_mfma_i32_16x16x32_i8(__builtin_bit_cast(long, ac[b]),
                                                                         __builtin_bit_cast(long, cw8[b]),
                                                                         i32x4_t{0, 0, 0, 0}, 0, 0, 0);
                const float4 da = *(const float4 *)&s_da[w][b][4 * q];
                acc[0] += (float)ci[0] * (sc[b] * da.x);
                acc[1] += (float)ci[1] * (sc[b] * da.y);
                acc[2] += (float)ci[2] * (sc[b] * da.z);
                acc[3] += (float)ci[3] * (sc[b] * da.w);
            }
        } else {
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                // one product per block: the other block's lanes contribute zero codes
                const uint4 b1 = codes_to_f16(make_uint2(cw[p].x, cw[p].y)), b2 = codes_to_f16(make_uint2(cw[p].z, cw[p].w));
                const uint4 b1f = sel4(first, b1, z4), b2f = sel4(first, b2, z4), b1s = sel4(first, z4, b1),
                            b2s = sel4(first, z4, b2);
                f32x4_t cf = {0.f, 0.f, 0.f, 0.f}, cs = {0.f, 0.f, 0.f, 0.f};
                cf = mfma16(a1h[p], b1f, cf);
                cs = mfma16(a1h[p], b1s, cs);
                cf = mfma16(a1l[p], b1f, cf);
                cs = mfma16(a1l[p], b1s, cs);
                cf = mfma16(a2h[p], b2f, cf);
                cs = mfma16(a2h[p], b2s, cs);
                cf = mfma16(a2l[p], b2f, cf);
                cs = mfma16(a2l[p], b2s, cs);
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] += sc[2 * p] * cf[r] + sc[2 * p + 1] * cs[r];
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) red[w][r][lane] = acc[r];
        __syncthreads();
        if (tid < 256) {
            // sum of the waves' partials for (sequence es, row slot er), in wave order
            const int sl = 16 * (es >> 2) + er, r = es & 3;
            float v = 0.f;
#pragma unroll
            for (int ww = 0; ww < KW; ++ww) v += red[ww][r][sl];
            if constexpr (EPI == EPI_STORE) {
                const int row = t * 16 + er;
                if (es < S && row < a.N) a.y[(size_t)es * a.ldy + row] = v;
            } else if constexpr (EPI == EPI_RESID) {
                const int row = t * 16 + er;
                float nv = 0.f;
                if (es < S) {
                    float *yp = a.y + (size_t)es * a.ldy + row;
                    nv = *yp + v;
                    *yp = nv;
                }
                if (a.ssq_mode == 2) {
                    const float ss = row16_sum(nv * nv);  // the 16 rows of the tile, one sequence per 16 lanes
                    if (er == 0 && es < S) a.ssq[t * kMaxSeq + es] = ss;
                }
            } else if constexpr (EPI == EPI_SWIGLU) {
                const float up = dpp_mov<0x128>(v);  // row_ror:8 -- slot er + 8 holds the up row of slot er
                if (er < 8 && es < S) {
                    // SwiGLU, [P1] section 5: (g * sigmoid(g)) * u with sigmoid(g) = 1 / (1 + exp(-g))
                    const float sig = 1.0f / (1.0f + __expf(-v));
                    const float act = (v * sig) * up;
                    const int unit = t * 8 + er;
                    if (a.y) a.y[(size_t)es * a.ldy + unit] = act;
                    uint16_t h, l;
                    split_one(act, h, l);
                    const size_t o = mfma_opnd_index(unit, es);
                    a.o_hi[o] = h;
                    a.o_lo[o] = l;
                }
            } else {  // EPI_LOGITS
                const int row = t * 16 + er;
                if (es < S && row < a.N) {
                    a.y[(size_t)es * a.ldy + row] = v;
                    if (!isfinite(v)) bad = 1;
                    if (v > best) {  // rows visited in increasing order: ties keep the lowest id
                        best = v;
                        besti = row;
                    }
                }
            }
        }
        __syncthreads();
        if constexpr (kStride) {
#pragma unroll
            for (int p = 0; p < NP; ++p) cw[p] = cn[p];
#pragma unroll
            for (int b = 0; b < NB; ++b) cw8[b] = cn8[b];
#pragma unroll
            for (int j = 0; j < NB; ++j) sc[j] = sn[j];
        }
    }

    if constexpr (EPI == EPI_LOGITS) {
        // per-workgroup greedy partial of each sequence: greatest value, lowest index on ties ([P4] "Sampling
        // order"); a non-finite logit latches a numerical failure ([P1] section 4)
        if (tid < 256) {
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) {
                const float ov = __shfl_xor(best, o, 64);
                const int oi = __shfl_xor(besti, o, 64);
                if (ov > best || (ov == best && oi < besti)) {
                    best = ov;
                    besti = oi;
                }
            }
            if (bad) atomicOr(a.status, kStatusNonFinite);
            if (er == 0 && es < S) {
                float *p = a.argpart + ((size_t)es * gridDim.x + blockIdx.x) * 2;
                p[0] = best;
                p[1] = __int_as_float(besti);
            }
        }
    }
}

// Per-16-row sums of squares of the step's first residual stream (the embedding rows), as the residual
// epilogues leave them for later RMSNorms.  One workgroup per sequence.
__global__ __launch_bounds__(256) void ssq_prep_kernel(const float *x, int ldx, int K, float *ssq) {
    const int s = blockIdx.x;
    for (int k0 = threadIdx.x * 4; k0 < K; k0 += 1024) {
        const float4 v = *(const float4 *)(x + (size_t)s * ldx + k0);
        float ss = (v.x * v.x + v.y * v.y) + (v.z * v.z + v.w * v.w);
        // four threads hold a 16-row tile
        ss += dpp_mov<0xB1>(ss);
        ss += dpp_mov<0x4E>(ss);
        if ((threadIdx.x & 3) == 0) ssq[(k0 >> 4) * kMaxSeq + s] = ss;
    }
}

}  // namespace

bool gemv_mfma_supported(const GemvArgs &a, GemvEpi epi) {
    if (a.S < 2 || a.S > kMaxSeq || a.K % 32) return false;
    switch (epi) {
        case EPI_STORE:
        case EPI_LOGITS: return a.K == 1024;
        case EPI_SWIGLU: return a.K == 1024 && a.N % 8 == 0;
        case EPI_RESID: return (a.K == 1024 || a.K == 2048 || a.K == 3072) && a.N % 16 == 0;
    }
    return false;
}

hipError_t launch_ssq_prep(const float *x, int ldx, int S, int K, float *ssq, hipStream_t st) {
    if (S < 1 || S > kMaxSeq || K % 16) return hipErrorInvalidValue;
    hipLaunchKernelGGL(ssq_prep_kernel, dim3(S), dim3(256), 0, st, x, ldx, K, ssq);
    return hipGetLastError();
}

// The f16-operand or, for the q8 x q8 format (a.act8), the int8 form of one product.
template <int KW, int NB, int EPI>
void launch_form(const GemvArgs &a, dim3 grid, dim3 block, hipStream_t st) {
    if (a.act8)
        hipLaunchKernelGGL((gemv_mfma_kernel<KW, NB, EPI, true>), grid, block, 0, st, a);
    else
        hipLaunchKernelGGL((gemv_mfma_kernel<KW, NB, EPI, false>), grid, block, 0, st, a);
}

hipError_t launch_gemv_mfma(GemvEpi epi, const GemvArgs &a, hipStream_t st) {
    if (!gemv_mfma_supported(a, epi)) return hipErrorInvalidValue;
    switch (epi) {
        case EPI_STORE: {
            // one tile per workgroup while the tiles fit the compute units in one round (Q/K/V: 256 tiles,
            // measured 7.5 us against 8.8 us for two tiles per workgroup); two beyond that
            const int ntiles = (a.N + 15) / 16;
            launch_form<4, 8, EPI_STORE>(a, dim3(ntiles > 256 ? (ntiles + 1) / 2 : ntiles), dim3(256), st);
            break;
        }
        case EPI_SWIGLU: {
            // 384 tiles for the 3072-unit MLP: two per workgroup (one per workgroup, 384 workgroups on 256 compute
            // units, measured 11.4 us against 9.2 us)
            const int ntiles = a.N / 8;
            launch_form<4, 8, EPI_SWIGLU>(a, dim3(ntiles > 128 ? (ntiles + 1) / 2 : ntiles), dim3(256), st);
            break;
        }
        case EPI_RESID:
            switch (a.K) {
                case 1024: launch_form<16, 2, EPI_RESID>(a, dim3(a.N / 16), dim3(1024), st); break;
                case 2048: launch_form<16, 4, EPI_RESID>(a, dim3(a.N / 16), dim3(1024), st); break;
                default: launch_form<16, 6, EPI_RESID>(a, dim3(a.N / 16), dim3(1024), st); break;
            }
            break;
        case EPI_LOGITS: {
            const int ntiles = (a.N + 15) / 16;
            const int grid = ntiles < 512 ? ntiles : 512;
            hipLaunchKernelGGL((gemv_mfma_kernel<4, 8, EPI_LOGITS>), dim3(grid), dim3(256), 0, st, a);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            return launch_argmax_finalize(a.argpart, grid, a.S, a.argmax_out, a.len, a.commit_add, a.status, st);
        }
    }
    return hipGetLastError();
}

}  // namespace qw3
