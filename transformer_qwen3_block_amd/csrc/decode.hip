// Decode-path kernels for gfx950: weight-streaming GEMV (bf16 or Q8 with in-register dequant) with fused
// RMSNorm prologue and residual / SwiGLU / logits+argmax epilogues, split-context GQA attention with fused
// QK-Norm, RoPE and KV append, and the small embedding / bookkeeping kernels.
//
// Page titles used in citations:
//   [P1] "Scalar-Native Qwen3 Reference Runtime As The Numerical Authority"
//   [P4] "Portable WebAssembly Runtime Architecture for TinyRustLM"
#include <math.h>

#include "common.h"

namespace qw3 {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

// Widen the 16 int8 codes of a 16-byte load to f32.
__device__ __forceinline__ void unpack_i8x16(const uint4 &w, float (&o)[16]) {
    const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int b = 0; b < 4; ++b) o[4 * j + b] = (float)(int8_t)(d[j] >> (8 * b));
    }
}

__device__ __forceinline__ void unpack_bf16x8(const uint4 &w, float (&o)[8]) {
    const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        o[2 * j] = bf16_lo(d[j]);
        o[2 * j + 1] = bf16_hi(d[j]);
    }
}

// ---------------------------------------------------------------------------------------------------
// GEMV: y[s][unit] = epilogue( sum_k W[row][k] * xhat[s][k] ) for S input vectors.
//
// One wave (64 lanes) owns R output units; the lanes split K in 16-byte slices (8 bf16 or 16 Q8 codes),
// so every weight row is read once, fully coalesced, and reduced across the wave at the end.  The input
// vectors (RMS-normalised when norm_w is given, [P1] section 2 items 1 and 6) are staged in LDS in
// chunks of KC columns.  Q8 slices are dequantised in registers and the per-32 scale is applied to the
// slice's partial sum.  Each output element is produced by exactly one wave: no float atomics.
// ---------------------------------------------------------------------------------------------------
template <int Q8, int SM, int R, int EPI>
__global__ __launch_bounds__(256) void gemv_kernel(GemvArgs a, int KC) {
    constexpr int E = Q8 ? 16 : 8;
    constexpr int RPU = (EPI == EPI_SWIGLU) ? 2 : 1;
    constexpr int NR = R * RPU;
    extern __shared__ float xs[];  // [S][KC]
    __shared__ float red[4][kMaxSeq];
    __shared__ float inv_s[kMaxSeq];
    __shared__ float bv[4][kMaxSeq];
    __shared__ int bi[4][kMaxSeq];
    __shared__ int is_last;
    __shared__ int bad;

    const int S = a.S, K = a.K;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int unit0 = (blockIdx.x * 4 + wave) * R;

    if (a.norm_w) {
        for (int s = 0; s < S; ++s) {
            float ss = 0.f;
            const float *xr = a.x + (size_t)s * a.ldx;
            for (int k = tid; k < K; k += 256) {
                float v = xr[k];
                ss += v * v;
            }
            ss = wave_sum(ss);
            if (lane == 0) red[wave][s] = ss;
        }
        __syncthreads();
        if (tid < S) {
            float ss = (red[0][tid] + red[1][tid]) + (red[2][tid] + red[3][tid]);
            inv_s[tid] = 1.0f / sqrtf(ss / (float)K + a.eps);
        }
        __syncthreads();
    }

    long long row[NR];
    bool valid[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int unit = unit0 + r;
        valid[r] = unit < a.N;
#pragma unroll
        for (int u = 0; u < RPU; ++u) row[r * RPU + u] = valid[r] ? (long long)unit + (long long)u * a.N : 0;
    }

    float acc[NR][SM];
#pragma unroll
    for (int j = 0; j < NR; ++j)
#pragma unroll
        for (int s = 0; s < SM; ++s) acc[j][s] = 0.f;

    const int kblocks = K / 32;
    for (int k0 = 0; k0 < K; k0 += KC) {
        const int kc = min(KC, K - k0);
        __syncthreads();
        for (int s = 0; s < S; ++s) {
            const float *xr = a.x + (size_t)s * a.ldx + k0;
            for (int k = tid * 4; k < kc; k += 1024) {
                float4 v = *(const float4 *)(xr + k);
                if (a.norm_w) {
                    const float4 w = *(const float4 *)(a.norm_w + k0 + k);
                    const float inv = inv_s[s];
                    v.x = w.x * (v.x * inv);
                    v.y = w.y * (v.y * inv);
                    v.z = w.z * (v.z * inv);
                    v.w = w.w * (v.w * inv);
                }
                *(float4 *)(xs + s * KC + k) = v;
            }
        }
        __syncthreads();
        for (int sl = lane; sl < kc / E; sl += 64) {
            const int kk = k0 + sl * E;
            uint4 wv[NR];
            float sc[NR];
#pragma unroll
            for (int j = 0; j < NR; ++j) {
                if (valid[j / RPU]) {
                    const char *base = (const char *)a.w + (size_t)(row[j] * (long long)K + kk) * (Q8 ? 1 : 2);
                    wv[j] = load_nt16(base);
                    if (Q8) sc[j] = a.scales[row[j] * kblocks + (kk >> 5)];
                } else {
                    wv[j] = make_uint4(0, 0, 0, 0);
                    sc[j] = 0.f;
                }
            }
            float wf[NR][E];
#pragma unroll
            for (int j = 0; j < NR; ++j) {
                if constexpr (Q8) {
                    unpack_i8x16(wv[j], wf[j]);
                } else {
                    unpack_bf16x8(wv[j], wf[j]);
                }
            }
#pragma unroll
            for (int s = 0; s < SM; ++s) {
                if (s < S) {
                    float xv[E];
                    const float4 *xp = (const float4 *)(xs + s * KC + sl * E);
#pragma unroll
                    for (int q = 0; q < E / 4; ++q) {
                        float4 t = xp[q];
                        xv[4 * q] = t.x;
                        xv[4 * q + 1] = t.y;
                        xv[4 * q + 2] = t.z;
                        xv[4 * q + 3] = t.w;
                    }
#pragma unroll
                    for (int j = 0; j < NR; ++j) {
                        if constexpr (Q8) {
                            float d = 0.f;
#pragma unroll
                            for (int e = 0; e < E; ++e) d += wf[j][e] * xv[e];
                            acc[j][s] += d * sc[j];
                        } else {
#pragma unroll
                            for (int e = 0; e < E; ++e) acc[j][s] += wf[j][e] * xv[e];
                        }
                    }
                }
            }
        }
    }

#pragma unroll
    for (int j = 0; j < NR; ++j)
#pragma unroll
        for (int s = 0; s < SM; ++s) acc[j][s] = wave_sum(acc[j][s]);

    if constexpr (EPI == EPI_LOGITS) {
        // logits, then the greedy choice: greatest value, lowest index on ties ([P4] "Sampling order");
        // a non-finite logit latches a numerical failure ([P1] section 4).
        if (tid == 0) bad = 0;
        __syncthreads();
        int my_bad = 0;
#pragma unroll
        for (int s = 0; s < SM; ++s) {
            if (s < S) {
                float best = -INFINITY;
                int besti = 0x7fffffff;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    if (valid[r]) {
                        const float v = acc[r][s];
                        if (lane == 0) a.y[(size_t)s * a.ldy + unit0 + r] = v;
                        if (!isfinite(v)) my_bad = 1;
                        if (v > best) {
                            best = v;
                            besti = unit0 + r;
                        }
                    }
                }
                if (lane == 0) {
                    bv[wave][s] = best;
                    bi[wave][s] = besti;
                }
            }
        }
        if (lane == 0 && my_bad) bad = 1;
        __syncthreads();
        if (tid < S) {
            float best = -INFINITY;
            int besti = 0x7fffffff;
            for (int w = 0; w < 4; ++w) {
                const float v = bv[w][tid];
                const int i = bi[w][tid];
                if (v > best || (v == best && i < besti)) {
                    best = v;
                    besti = i;
                }
            }
            float *p = a.argpart + ((size_t)tid * gridDim.x + blockIdx.x) * 2;
            p[0] = best;
            p[1] = __int_as_float(besti);
        }
        if (tid == 0 && bad) atomicOr(a.status, 1);
        __threadfence();
        __syncthreads();
        if (tid == 0) is_last = (atomicAdd(a.counter, 1u) == gridDim.x - 1);
        __syncthreads();
        if (!is_last) return;
        __threadfence();
        for (int s = 0; s < S; ++s) {
            float best = -INFINITY;
            int besti = 0x7fffffff;
            for (int b = tid; b < (int)gridDim.x; b += 256) {
                const float *p = a.argpart + ((size_t)s * gridDim.x + b) * 2;
                const float v = __builtin_nontemporal_load(p);
                const int i = __float_as_int(__builtin_nontemporal_load(p + 1));
                if (v > best || (v == best && i < besti)) {
                    best = v;
                    besti = i;
                }
            }
            // wave then block reduction of (value, index)
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) {
                const float ov = __shfl_xor(best, o, 64);
                const int oi = __shfl_xor(besti, o, 64);
                if (ov > best || (ov == best && oi < besti)) {
                    best = ov;
                    besti = oi;
                }
            }
            if (lane == 0) {
                bv[wave][s] = best;
                bi[wave][s] = besti;
            }
        }
        __syncthreads();
        if (tid < S) {
            float best = -INFINITY;
            int besti = 0x7fffffff;
            for (int w = 0; w < 4; ++w) {
                const float v = bv[w][tid];
                const int i = bi[w][tid];
                if (v > best || (v == best && i < besti)) {
                    best = v;
                    besti = i;
                }
            }
            // all logits NaN: no index qualifies; report 0 (the status word carries the failure)
            if (a.argmax_out) a.argmax_out[tid] = besti == 0x7fffffff ? 0 : besti;
            // commit: the appended positions become valid only now ([P4] "Cancellation")
            if (a.len) a.len[tid] += a.commit_add;
        }
        if (tid == 0) *a.counter = 0u;
    } else {
        if (lane == 0) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                if (!valid[r]) continue;
                const int unit = unit0 + r;
#pragma unroll
                for (int s = 0; s < SM; ++s) {
                    if (s >= S) continue;
                    float *yp = a.y + (size_t)s * a.ldy + unit;
                    if constexpr (EPI == EPI_STORE) {
                        *yp = acc[r][s];
                    } else if constexpr (EPI == EPI_RESID) {
                        *yp = *yp + acc[r][s];
                    } else {
                        // SwiGLU, [P1] section 5: (g * sigmoid(g)) * u with sigmoid(g) = 1 / (1 + exp(-g))
                        const float g = acc[2 * r][s], u = acc[2 * r + 1][s];
                        const float sig = 1.0f / (1.0f + __expf(-g));
                        *yp = (g * sig) * u;
                    }
                }
            }
        }
    }
}

template <int Q8, int SM, int EPI>
hipError_t gemv_dispatch_r(int R, const GemvArgs &a, int KC, size_t lds, hipStream_t st) {
    const int units_per_block = 4 * R;
    const int grid = (a.N + units_per_block - 1) / units_per_block;
    switch (R) {
        case 1: hipLaunchKernelGGL((gemv_kernel<Q8, SM, 1, EPI>), dim3(grid), dim3(256), lds, st, a, KC); break;
        case 2: hipLaunchKernelGGL((gemv_kernel<Q8, SM, 2, EPI>), dim3(grid), dim3(256), lds, st, a, KC); break;
        case 4:
            if constexpr (SM == 1 || EPI == EPI_LOGITS) {
                hipLaunchKernelGGL((gemv_kernel<Q8, SM, 4, EPI>), dim3(grid), dim3(256), lds, st, a, KC);
                break;
            }
            return hipErrorInvalidValue;
        case 8:
            if constexpr (SM == 1 && EPI != EPI_SWIGLU) {
                hipLaunchKernelGGL((gemv_kernel<Q8, SM, 8, EPI>), dim3(grid), dim3(256), lds, st, a, KC);
                break;
            }
            return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int Q8, int EPI>
hipError_t gemv_dispatch_s(const GemvArgs &a, hipStream_t st) {
    const int E = Q8 ? 16 : 8;
    // LDS budget for the staged input vectors: whole K when it fits in 64 KB, else chunks that are
    // multiples of one wave's slice span (64 * E columns).
    int KC = a.K;
    const int budget = 16384;  // floats
    if (a.S * KC > budget) {
        KC = (budget / a.S) / (64 * E) * (64 * E);
        if (KC < 64 * E) KC = 64 * E;
    }
    const size_t lds = (size_t)a.S * KC * sizeof(float);
    // units per wave: as many as keep >= ~2 workgroups per CU
    int R = 1;
    if (a.S == 1) {
        const int maxR = (EPI == EPI_SWIGLU) ? 4 : 8;
        while (R < maxR && (a.N + 8 * R - 1) / (8 * R) >= 512) R *= 2;
        if (EPI == EPI_LOGITS) {
            while (R < maxR && (a.N + 4 * R - 1) / (4 * R) > kLmMaxBlocks) R *= 2;
            if ((a.N + 4 * R - 1) / (4 * R) > kLmMaxBlocks) return hipErrorInvalidValue;
        }
        return gemv_dispatch_r<Q8, 1, EPI>(R, a, KC, lds, st);
    }
    if (EPI != EPI_SWIGLU && (a.N + 7) / 8 >= 256) R = 2;
    if (EPI == EPI_LOGITS) {
        while (R < 4 && (a.N + 4 * R - 1) / (4 * R) > kLmMaxBlocks) R *= 2;
        if ((a.N + 4 * R - 1) / (4 * R) > kLmMaxBlocks) return hipErrorInvalidValue;
    }
    return gemv_dispatch_r<Q8, kMaxSeq, EPI>(R, a, KC, lds, st);
}

// ---------------------------------------------------------------------------------------------------
// Decode attention for one token per sequence, split over the context.
//
// Grid (n_split, HKV, S); the workgroup of (split, kv head g, seq s) serves the G query heads that read
// KV head g (h_kv = floor(h_q / G), [P1] section 2 item 5).  It first applies QK-Norm ([P1] item 3) and
// RoPE ([P1] item 4, pairs (i, i+64), angles from the position's table row) to its query heads; the
// workgroup whose split holds the new position also normalises and rotates the new key, rounds key and
// value to bf16 and appends them to the cache ([P1] section 6).  Each wave then streams 16-position
// groups of K and V (1 KB per load instruction, 16 lanes per position, 8 dims per lane), keeping an online
// softmax (running max, running sum, rescaled accumulator) in log2 units.  Wave states are merged in LDS
// and written as the split's partial; the last workgroup to finish a (seq, kv head) merges the splits in
// split order, so the result does not depend on completion order.
// ---------------------------------------------------------------------------------------------------
template <int G>
__global__ __launch_bounds__(256) void attn_decode_kernel(AttnDecodeArgs a) {
    const int split = blockIdx.x, kvh = blockIdx.y, s = blockIdx.z;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    __shared__ float qs[G][kHeadDim];
    __shared__ float knew[kHeadDim];
    __shared__ float red[4];
    __shared__ float wm[4][G], wl[4][G];
    __shared__ float wacc[4][G][kHeadDim];
    __shared__ int is_last;

    const int pos = a.len[s];
    const int n = pos + 1;
    int chunk = (n + a.n_split - 1) / a.n_split;
    chunk = (chunk + 15) & ~15;
    const int start = split * chunk;
    const int end = min(n, start + chunk);
    const float *qkv = a.qkv + (size_t)s * a.ldqkv;
    const float *cosr = a.rope_cos + (size_t)pos * (kHeadDim / 2);
    const float *sinr = a.rope_sin + (size_t)pos * (kHeadDim / 2);
    const int q_dim = a.HQ * kHeadDim;

    // ---- QK-Norm + RoPE of this group's query heads (two heads per pass, 128 threads each)
    for (int hb = 0; hb < G; hb += 2) {
        const int h = hb + (tid >> 7), d = tid & 127;
        const bool act = h < G;
        const float v = act ? qkv[(size_t)(kvh * G + h) * kHeadDim + d] : 0.f;
        const float ss = wave_sum(v * v);
        if (lane == 0) red[wave] = ss;
        __syncthreads();
        const int w0 = (tid >> 7) * 2;
        const float inv = 1.0f / sqrtf((red[w0] + red[w0 + 1]) / (float)kHeadDim + a.eps);
        if (act) qs[h][d] = a.q_norm[d] * (v * inv);
        __syncthreads();
        float r = 0.f;
        if (act) {
            const int i = d & 63;
            const float c = cosr[i], sn = sinr[i];
            const float x1 = qs[h][i], x2 = qs[h][i + 64];
            r = d < 64 ? x1 * c - x2 * sn : x2 * c + x1 * sn;
        }
        __syncthreads();
        if (act) qs[h][d] = r;
        __syncthreads();
    }

    const size_t head_off = (size_t)s * a.seq_stride + (size_t)kvh * a.max_ctx * kHeadDim;
    const uint16_t *kb = a.kcache + head_off;
    const uint16_t *vb = a.vcache + head_off;

    // ---- append the new key/value (only the workgroup whose split holds the new position)
    if (pos >= start && pos < end) {
        const int d = tid & 127;
        const bool is_k = tid < 128;
        const float v = is_k ? qkv[q_dim + kvh * kHeadDim + d] : qkv[q_dim + (a.HKV + kvh) * kHeadDim + d];
        const float ss = wave_sum(v * v);
        if (lane == 0) red[wave] = ss;
        __syncthreads();
        float out = v;
        if (is_k) {
            const float inv = 1.0f / sqrtf((red[0] + red[1]) / (float)kHeadDim + a.eps);
            knew[d] = a.k_norm[d] * (v * inv);
        }
        __syncthreads();
        if (is_k) {
            const int i = d & 63;
            const float c = cosr[i], sn = sinr[i];
            const float x1 = knew[i], x2 = knew[i + 64];
            out = d < 64 ? x1 * c - x2 * sn : x2 * c + x1 * sn;
        }
        uint16_t *dst = (uint16_t *)(is_k ? kb : vb) + (size_t)pos * kHeadDim + d;
        *dst = f32_to_bf16(out);
        __threadfence();
        __syncthreads();
    }

    // ---- stream this split's positions
    const int dsub = (lane & 15) * 8;
    const int prow = lane >> 4;
    float qr[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) qr[h][e] = qs[h][dsub + e];
    const float sl2 = (1.0f / sqrtf((float)kHeadDim)) * kLog2e;
    float m[G], l[G], acc[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
    }

    for (int j0 = start + 16 * wave; j0 < end; j0 += 64) {
        uint4 kr[4], vr[4];
        bool val[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int p = j0 + 4 * i + prow;
            val[i] = p < end;
            if (val[i]) {
                kr[i] = load_nt16(kb + (size_t)p * kHeadDim + dsub);
                vr[i] = load_nt16(vb + (size_t)p * kHeadDim + dsub);
            } else {
                kr[i] = make_uint4(0, 0, 0, 0);
                vr[i] = make_uint4(0, 0, 0, 0);
            }
        }
        float sc[G][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float kf[8];
            unpack_bf16x8(kr[i], kf);
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float d = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) d += qr[h][e] * kf[e];
                d += __shfl_xor(d, 8, 64);
                d += __shfl_xor(d, 4, 64);
                d += __shfl_xor(d, 2, 64);
                d += __shfl_xor(d, 1, 64);
                sc[h][i] = val[i] ? d * sl2 : -INFINITY;
            }
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float tm = fmaxf(fmaxf(sc[h][0], sc[h][1]), fmaxf(sc[h][2], sc[h][3]));
            tm = fmaxf(tm, __shfl_xor(tm, 16, 64));
            tm = fmaxf(tm, __shfl_xor(tm, 32, 64));
            const float mn = fmaxf(m[h], tm);
            const float alpha = exp2f(m[h] - mn);
            l[h] *= alpha;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] *= alpha;
            m[h] = mn;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float vf[8];
            unpack_bf16x8(vr[i], vf);
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float p = exp2f(sc[h][i] - m[h]);
                l[h] += p;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[h][e] += p * vf[e];
            }
        }
    }

    // ---- merge the four position rows of the wave, then the four waves
#pragma unroll
    for (int h = 0; h < G; ++h) {
        l[h] += __shfl_xor(l[h], 16, 64);
        l[h] += __shfl_xor(l[h], 32, 64);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            acc[h][e] += __shfl_xor(acc[h][e], 16, 64);
            acc[h][e] += __shfl_xor(acc[h][e], 32, 64);
        }
        if (lane < 16) {
#pragma unroll
            for (int e = 0; e < 8; ++e) wacc[wave][h][dsub + e] = acc[h][e];
        }
        if (lane == 0) {
            wm[wave][h] = m[h];
            wl[wave][h] = l[h];
        }
    }
    __syncthreads();
    for (int t = tid; t < G * kHeadDim; t += 256) {
        const int h = t >> 7, d = t & 127;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, wm[w][h]);
        float L = 0.f, O = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float f = exp2f(wm[w][h] - M);
                L += f * wl[w][h];
                O += f * wacc[w][h][d];
            }
        }
        float *p = a.part + (((size_t)s * a.HQ + kvh * G + h) * kMaxSplit + split) * kPartStride;
        if (d == 0) {
            p[0] = M;
            p[1] = L;
        }
        p[2 + d] = O;
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) is_last = (atomicAdd(a.counters + s * a.HKV + kvh, 1u) == gridDim.x - 1);
    __syncthreads();
    if (!is_last) return;
    __threadfence();
    for (int t = tid; t < G * kHeadDim; t += 256) {
        const int h = t >> 7, d = t & 127;
        const float *p0 = a.part + (((size_t)s * a.HQ + kvh * G + h) * kMaxSplit) * kPartStride;
        float M = -INFINITY;
        for (int sp = 0; sp < a.n_split; ++sp) M = fmaxf(M, __builtin_nontemporal_load(p0 + sp * kPartStride));
        float L = 0.f, O = 0.f;
        for (int sp = 0; sp < a.n_split; ++sp) {
            const float *p = p0 + sp * kPartStride;
            const float f = exp2f(__builtin_nontemporal_load(p) - M);
            L += f * __builtin_nontemporal_load(p + 1);
            O += f * __builtin_nontemporal_load(p + 2 + d);
        }
        a.out[(size_t)s * a.ldo + (kvh * G + h) * kHeadDim + d] = O / L;
    }
    if (tid == 0) a.counters[s * a.HKV + kvh] = 0u;
}

// Embedding: x[s] = row tokens[s] of the table, widened (bf16) or dequantised (code * scale).
template <int Q8>
__global__ void embed_kernel(const void *table, const float *scales, int H, const int *tokens, float *x,
                             int *status, int vocab) {
    const int s = blockIdx.y;
    const int k = blockIdx.x * blockDim.x + threadIdx.x;
    int tok = tokens[s];
    if (tok < 0 || tok >= vocab) {
        if (k == 0) atomicOr(status, 2);
        tok = 0;
    }
    if (k >= H) return;
    const size_t i = (size_t)tok * H + k;
    float v;
    if (Q8)
        v = (float)((const int8_t *)table)[i] * scales[i >> 5];
    else
        v = bf16_to_f32(((const uint16_t *)table)[i]);
    x[(size_t)s * H + k] = v;
}

struct LenVals {
    int v[kMaxSeq];
};

__global__ void set_lens_kernel(int *len, int n, LenVals vals, int mask, int *status, int clear_status) {
    const int t = threadIdx.x;
    if (t < n && (mask >> t) & 1) len[t] = vals.v[t];
    if (t == 0 && clear_status) *status = 0;
}

__global__ void commit_kernel(int *len, int n, int add) {
    const int t = threadIdx.x;
    if (t < n) len[t] += add;
}

template <int Q8>
__global__ void dequant_kernel(const void *w, const float *scales, long long total, int cols, float *out) {
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total) return;
    if (Q8)
        out[i] = (float)((const int8_t *)w)[i] * scales[i >> 5];
    else
        out[i] = bf16_to_f32(((const uint16_t *)w)[i]);
}

}  // namespace

hipError_t launch_gemv(bool q8, GemvEpi epi, const GemvArgs &a, hipStream_t st) {
    if (a.S < 1 || a.S > kMaxSeq || a.K % (q8 ? 1024 : 512)) return hipErrorInvalidValue;
#define QW3_GEMV_EPI(Q)                                                       \
    switch (epi) {                                                            \
        case EPI_STORE: return gemv_dispatch_s<Q, EPI_STORE>(a, st);          \
        case EPI_RESID: return gemv_dispatch_s<Q, EPI_RESID>(a, st);          \
        case EPI_SWIGLU: return gemv_dispatch_s<Q, EPI_SWIGLU>(a, st);        \
        case EPI_LOGITS: return gemv_dispatch_s<Q, EPI_LOGITS>(a, st);        \
    }
    if (q8) {
        QW3_GEMV_EPI(1)
    } else {
        QW3_GEMV_EPI(0)
    }
#undef QW3_GEMV_EPI
    return hipErrorInvalidValue;
}

hipError_t launch_attn_decode(int G, const AttnDecodeArgs &a, hipStream_t st) {
    if (a.n_split < 1 || a.n_split > kMaxSplit) return hipErrorInvalidValue;
    const dim3 grid(a.n_split, a.HKV, a.S);
    switch (G) {
        case 1: hipLaunchKernelGGL(attn_decode_kernel<1>, grid, dim3(256), 0, st, a); break;
        case 2: hipLaunchKernelGGL(attn_decode_kernel<2>, grid, dim3(256), 0, st, a); break;
        case 4: hipLaunchKernelGGL(attn_decode_kernel<4>, grid, dim3(256), 0, st, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_embed(bool q8, const void *table, const float *scales, int H, const int *tokens, int S, float *x,
                        int *status, int vocab, hipStream_t st) {
    const dim3 grid((H + 255) / 256, S);
    if (q8)
        hipLaunchKernelGGL(embed_kernel<1>, grid, dim3(256), 0, st, table, scales, H, tokens, x, status, vocab);
    else
        hipLaunchKernelGGL(embed_kernel<0>, grid, dim3(256), 0, st, table, scales, H, tokens, x, status, vocab);
    return hipGetLastError();
}

hipError_t launch_set_lens(int *len_dev, int n, const int *vals, int mask, int *status, int clear_status,
                           hipStream_t st) {
    LenVals v{};
    for (int i = 0; i < n && i < kMaxSeq; ++i) v.v[i] = vals[i];
    hipLaunchKernelGGL(set_lens_kernel, dim3(1), dim3(64), 0, st, len_dev, n, v, mask, status, clear_status);
    return hipGetLastError();
}

hipError_t launch_commit(int *len_dev, int n, int add, hipStream_t st) {
    hipLaunchKernelGGL(commit_kernel, dim3(1), dim3(64), 0, st, len_dev, n, add);
    return hipGetLastError();
}

hipError_t launch_dequant(bool q8, const void *w, const float *scales, long long rows, int cols, float *out,
                          hipStream_t st) {
    const long long total = rows * cols;
    const unsigned grid = (unsigned)((total + 255) / 256);
    if (q8)
        hipLaunchKernelGGL(dequant_kernel<1>, dim3(grid), dim3(256), 0, st, w, scales, total, cols, out);
    else
        hipLaunchKernelGGL(dequant_kernel<0>, dim3(grid), dim3(256), 0, st, w, scales, total, cols, out);
    return hipGetLastError();
}

}  // namespace qw3
