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
// One wave (64 lanes) owns a group of R output units at a time; the lanes split K in 16-byte slices
// (8 bf16 or 16 Q8 codes, KS slices per lane per chunk of KC = KS*64*E columns), so every weight row is
// read once, fully coalesced, and reduced across the wave.  Weight loads never wait for activations: the
// first group's loads are issued before the input staging, and when the inputs fit in LDS in one chunk a
// wave walks its groups (grid-stride) with the next group's weights in flight while it computes the
// current one.  The inputs (RMS-normalised when norm_w is given, [P1] section 2 items 1 and 6) are staged
// in LDS.  Q8 slices are dequantised in registers and the per-32 scale multiplies the slice's partial sum.
// Each output element is produced by exactly one wave: no float atomics.
// ---------------------------------------------------------------------------------------------------
template <int Q8, int NR, int KS>
__device__ __forceinline__ void gemv_load(const GemvArgs &a, const long long (&row)[NR], bool ok, int k0, int lane,
                                          uint4 (&wv)[NR][KS], float (&sc)[NR][KS]) {
    constexpr int E = Q8 ? 16 : 8;
    const int kblocks = a.K / 32;
#pragma unroll
    for (int j = 0; j < NR; ++j) {
#pragma unroll
        for (int t = 0; t < KS; ++t) {
            const int kk = k0 + (lane + 64 * t) * E;
            if (ok) {
                wv[j][t] = load_nt16((const char *)a.w + (size_t)(row[j] * (long long)a.K + kk) * (Q8 ? 1 : 2));
                sc[j][t] = Q8 ? a.scales[row[j] * kblocks + (kk >> 5)] : 0.f;
            } else {
                wv[j][t] = make_uint4(0, 0, 0, 0);
                sc[j][t] = 0.f;
            }
        }
    }
}

// Rows of unit group g (SwiGLU: gate row u and up row u + N per unit).  Rows past the end are clamped to
// the last unit so loads stay in bounds; their results are never stored.
template <int R, int RPU>
__device__ __forceinline__ void gemv_rows(const GemvArgs &a, int g, long long (&row)[R * RPU]) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int unit = min(g * R + r, a.N - 1);
#pragma unroll
        for (int u = 0; u < RPU; ++u) row[r * RPU + u] = (long long)unit + (long long)u * a.N;
    }
}

template <int Q8, int SM, int NR, int KS>
__device__ __forceinline__ void gemv_dot(const uint4 (&wv)[NR][KS], const float (&sc)[NR][KS], const float *xs, int KC,
                                         int S, int lane, float (&acc)[NR][SM]) {
    constexpr int E = Q8 ? 16 : 8;
#pragma unroll
    for (int t = 0; t < KS; ++t) {
        const int sl = lane + 64 * t;
#pragma unroll
        for (int s = 0; s < SM; ++s) {
            if (s < S) {
                float xv[E];
                const float4 *xp = (const float4 *)(xs + s * KC + sl * E);
#pragma unroll
                for (int q = 0; q < E / 4; ++q) {
                    const float4 v = xp[q];
                    xv[4 * q] = v.x;
                    xv[4 * q + 1] = v.y;
                    xv[4 * q + 2] = v.z;
                    xv[4 * q + 3] = v.w;
                }
#pragma unroll
                for (int j = 0; j < NR; ++j) {
                    float wf[E];
                    if constexpr (Q8) {
                        unpack_i8x16(wv[j][t], wf);
                        float d = 0.f;
#pragma unroll
                        for (int e = 0; e < E; ++e) d += wf[e] * xv[e];
                        acc[j][s] += d * sc[j][t];
                    } else {
                        unpack_bf16x8(wv[j][t], wf);
#pragma unroll
                        for (int e = 0; e < E; ++e) acc[j][s] += wf[e] * xv[e];
                    }
                }
            }
        }
    }
}

template <int Q8, int SM, int R, int EPI, int KS>
__global__ __launch_bounds__(256) void gemv_kernel(GemvArgs a, int KC) {
    constexpr int RPU = (EPI == EPI_SWIGLU) ? 2 : 1;
    constexpr int NR = R * RPU;
    extern __shared__ float xs[];  // [S][KC]
    __shared__ float red[4][kMaxSeq];
    __shared__ float inv_s[kMaxSeq];
    __shared__ float bv[4][kMaxSeq];
    __shared__ int bi[4][kMaxSeq];

    const int S = a.S, K = a.K;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int n_groups = (a.N + R - 1) / R;
    const int gstride = gridDim.x * 4;
    int g = blockIdx.x * 4 + wave;
    const bool single = KC >= K;

    long long row[NR];
    uint4 wv[NR][KS];
    float sc[NR][KS];
    gemv_rows<R, RPU>(a, g, row);
    gemv_load<Q8, NR, KS>(a, row, g < n_groups, 0, lane, wv, sc);

    // running greedy choice of this wave (logits epilogue)
    float best[SM];
    int besti[SM];
    int my_bad = 0;
#pragma unroll
    for (int s = 0; s < SM; ++s) {
        best[s] = -INFINITY;
        besti[s] = 0x7fffffff;
    }

    auto epilogue = [&](int grp, float (&acc)[NR][SM]) {
        if constexpr (EPI == EPI_LOGITS && SM == 1 && NR == 4) {
            // the four rows' lane partials folded at once: lane row r ends up with row r's logit (the same
            // reduction tree for every row, so equal rows give equal logits); each lane row keeps its own
            // greedy choice over the rows it sees, in increasing order, and the rows are combined at the end
            const float v = row16_sum(swap16_sum(swap32_sum(acc[0][0], acc[2][0]), swap32_sum(acc[1][0], acc[3][0])));
            const int unit = grp * R + (lane >> 4);
            if (unit < a.N) {
                if ((lane & 15) == 0) a.y[unit] = v;
                if (!isfinite(v)) my_bad = 1;
                if (v > best[0]) {
                    best[0] = v;
                    besti[0] = unit;
                }
            }
            return;
        }
#pragma unroll
        for (int j = 0; j < NR; ++j)
#pragma unroll
            for (int s = 0; s < SM; ++s) acc[j][s] = wave_sum_fast(acc[j][s]);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int unit = grp * R + r;
            if (unit >= a.N) continue;
#pragma unroll
            for (int s = 0; s < SM; ++s) {
                if (s >= S) continue;
                float *yp = a.y + (size_t)s * a.ldy + unit;
                if constexpr (EPI == EPI_LOGITS) {
                    const float v = acc[r][s];
                    if (lane == 0) *yp = v;
                    if (!isfinite(v)) my_bad = 1;
                    if (v > best[s]) {  // units visited in increasing order: ties keep the lowest id
                        best[s] = v;
                        besti[s] = unit;
                    }
                } else if (lane == 0) {
                    if constexpr (EPI == EPI_STORE) {
                        *yp = acc[r][s];
                    } else if constexpr (EPI == EPI_RESID) {
                        *yp = *yp + acc[r][s];
                    } else {
                        // SwiGLU, [P1] section 5: (g * sigmoid(g)) * u with sigmoid(g) = 1 / (1 + exp(-g))
                        const float gt = acc[2 * r][s], up = acc[2 * r + 1][s];
                        const float sig = 1.0f / (1.0f + __expf(-gt));
                        *yp = (gt * sig) * up;
                    }
                }
            }
        }
    };

    if (single) {
        // stage all inputs once: raw values to LDS while summing squares, then normalise in place
        for (int s = 0; s < S; ++s) {
            const float *xr = a.x + (size_t)s * a.ldx;
            float ss = 0.f;
            for (int k = tid * 4; k < K; k += 1024) {
                const float4 v = *(const float4 *)(xr + k);
                ss += (v.x * v.x + v.y * v.y) + (v.z * v.z + v.w * v.w);
                *(float4 *)(xs + s * KC + k) = v;
            }
            if (a.norm_w) {
                ss = wave_sum(ss);
                if (lane == 0) red[wave][s] = ss;
            }
        }
        if (a.norm_w) {
            __syncthreads();
            if (tid < S) {
                const float ss = (red[0][tid] + red[1][tid]) + (red[2][tid] + red[3][tid]);
                inv_s[tid] = 1.0f / sqrtf(ss / (float)K + a.eps);
            }
            __syncthreads();
            for (int s = 0; s < S; ++s) {
                const float inv = inv_s[s];
                for (int k = tid * 4; k < K; k += 1024) {
                    float4 v = *(float4 *)(xs + s * KC + k);
                    const float4 w = *(const float4 *)(a.norm_w + k);
                    v.x = w.x * (v.x * inv);
                    v.y = w.y * (v.y * inv);
                    v.z = w.z * (v.z * inv);
                    v.w = w.w * (v.w * inv);
                    *(float4 *)(xs + s * KC + k) = v;
                }
            }
        }
        __syncthreads();
        while (g < n_groups) {
            const int gn = g + gstride;
            long long rn[NR];
            uint4 wn[NR][KS];
            float sn[NR][KS];
            gemv_rows<R, RPU>(a, gn, rn);
            gemv_load<Q8, NR, KS>(a, rn, gn < n_groups, 0, lane, wn, sn);
            float acc[NR][SM];
#pragma unroll
            for (int j = 0; j < NR; ++j)
#pragma unroll
                for (int s = 0; s < SM; ++s) acc[j][s] = 0.f;
            gemv_dot<Q8, SM, NR, KS>(wv, sc, xs, KC, S, lane, acc);
            epilogue(g, acc);
#pragma unroll
            for (int j = 0; j < NR; ++j) {
                row[j] = rn[j];
#pragma unroll
                for (int t = 0; t < KS; ++t) {
                    wv[j][t] = wn[j][t];
                    sc[j][t] = sn[j][t];
                }
            }
            g = gn;
        }
    } else {
        // inputs staged in chunks: one unit group per wave (the grid covers every group)
        if (a.norm_w) {
            for (int s = 0; s < S; ++s) {
                float ss = 0.f;
                const float *xr = a.x + (size_t)s * a.ldx;
                for (int k = tid; k < K; k += 256) {
                    const float v = xr[k];
                    ss += v * v;
                }
                ss = wave_sum(ss);
                if (lane == 0) red[wave][s] = ss;
            }
            __syncthreads();
            if (tid < S) {
                const float ss = (red[0][tid] + red[1][tid]) + (red[2][tid] + red[3][tid]);
                inv_s[tid] = 1.0f / sqrtf(ss / (float)K + a.eps);
            }
        }
        float acc[NR][SM];
#pragma unroll
        for (int j = 0; j < NR; ++j)
#pragma unroll
            for (int s = 0; s < SM; ++s) acc[j][s] = 0.f;
        for (int k0 = 0; k0 < K; k0 += KC) {
            if (k0) gemv_load<Q8, NR, KS>(a, row, g < n_groups, k0, lane, wv, sc);
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
            gemv_dot<Q8, SM, NR, KS>(wv, sc, xs, KC, S, lane, acc);
        }
        if (g < n_groups) epilogue(g, acc);
    }

    if constexpr (EPI == EPI_LOGITS) {
        // per-workgroup greedy partial: greatest value, lowest index on ties ([P4] "Sampling order"); a
        // non-finite logit latches a numerical failure ([P1] section 4).  The final choice over the
        // workgroups is made by argmax_finalize_kernel.
        if constexpr (SM == 1 && NR == 4) {  // the four lane rows' choices (see the epilogue)
#pragma unroll
            for (int o = 16; o <= 32; o <<= 1) {
                const float ov = __shfl_xor(best[0], o, 64);
                const int oi = __shfl_xor(besti[0], o, 64);
                if (ov > best[0] || (ov == best[0] && oi < besti[0])) {
                    best[0] = ov;
                    besti[0] = oi;
                }
            }
            my_bad = __any(my_bad) ? 1 : 0;
        }
        if (lane == 0) {
#pragma unroll
            for (int s = 0; s < SM; ++s) {
                if (s < S) {
                    bv[wave][s] = best[s];
                    bi[wave][s] = besti[s];
                }
            }
        }
        if (lane == 0 && my_bad) atomicOr(a.status, kStatusNonFinite);
        __syncthreads();
        if (tid < S) {
            float b = -INFINITY;
            int i0 = 0x7fffffff;
            for (int w = 0; w < 4; ++w) {
                const float v = bv[w][tid];
                const int i = bi[w][tid];
                if (v > b || (v == b && i < i0)) {
                    b = v;
                    i0 = i;
                }
            }
            float *p = a.argpart + ((size_t)tid * gridDim.x + blockIdx.x) * 2;
            p[0] = b;
            p[1] = __int_as_float(i0);
        }
    }
}

// Final greedy choice over the logits workgroups' partials (fixed order: lowest index wins ties), then the
// commit of the appended positions ([P4] "Cancellation": positions become valid only after the step).  A step
// that latched any failure in the status word (a non-finite logit, a token outside the vocabulary, a device
// wait that gave up) commits nothing, and neither does any later step until the handle is reset ([P1] section
// 4 "NaN/Inf Rejection": the generation loop stops at the failing step; section 8: completed steps stand).
__global__ __launch_bounds__(256) void argmax_finalize_kernel(const float *argpart, int nparts, int S, int *argmax_out,
                                                              int *len, int commit_add, const int *status) {
    // one workgroup per sequence (grid S); (value desc, id asc) is a total order, so the reduction order does not
    // change the result
    __shared__ float bv[4];
    __shared__ int bi[4];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int s = blockIdx.x;
    if (s >= S) return;
    const float2 *part = (const float2 *)argpart + (size_t)s * nparts;
    float best = -INFINITY;
    int besti = 0x7fffffff;
    auto take = [&](float2 p) {
        const float v = p.x;
        const int i = __float_as_int(p.y);
        if (v > best || (v == best && i < besti)) {
            best = v;
            besti = i;
        }
    };
    int b = tid;
    for (; b + 768 < nparts; b += 1024) {  // four partials in flight per thread
        const float2 p0 = part[b], p1 = part[b + 256], p2 = part[b + 512], p3 = part[b + 768];
        take(p0);
        take(p1);
        take(p2);
        take(p3);
    }
    for (; b < nparts; b += 256) take(part[b]);
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
        bv[wave] = best;
        bi[wave] = besti;
    }
    __syncthreads();
    if (tid == 0) {
        for (int w = 1; w < 4; ++w)
            if (bv[w] > bv[0] || (bv[w] == bv[0] && bi[w] < bi[0])) {
                bv[0] = bv[w];
                bi[0] = bi[w];
            }
        // all logits NaN: no index qualifies; report 0 (the status word carries the failure)
        if (argmax_out) argmax_out[s] = bi[0] == 0x7fffffff ? 0 : bi[0];
        if (len && *status == 0) len[s] += commit_add;
    }
}

template <int Q8, int SM, int R, int EPI>
hipError_t gemv_launch_ks(int KS, int grid, const GemvArgs &a, int KC, size_t lds, hipStream_t st) {
    switch (KS) {
        case 1: hipLaunchKernelGGL((gemv_kernel<Q8, SM, R, EPI, 1>), dim3(grid), dim3(256), lds, st, a, KC); break;
        case 2: hipLaunchKernelGGL((gemv_kernel<Q8, SM, R, EPI, 2>), dim3(grid), dim3(256), lds, st, a, KC); break;
        case 3:
            if constexpr (SM == 1) {
                hipLaunchKernelGGL((gemv_kernel<Q8, SM, R, EPI, 3>), dim3(grid), dim3(256), lds, st, a, KC);
                break;
            }
            return hipErrorInvalidValue;
        case 4:
            if constexpr (SM == 1 && R <= 2) {
                hipLaunchKernelGGL((gemv_kernel<Q8, SM, R, EPI, 4>), dim3(grid), dim3(256), lds, st, a, KC);
                break;
            }
            return hipErrorInvalidValue;
        case 6:
            if constexpr (SM == 1 && R <= 2 && !Q8) {
                hipLaunchKernelGGL((gemv_kernel<Q8, SM, R, EPI, 6>), dim3(grid), dim3(256), lds, st, a, KC);
                break;
            }
            return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int Q8, int SM, int EPI>
hipError_t gemv_launch_r(int R, int KS, int grid, const GemvArgs &a, int KC, size_t lds, hipStream_t st) {
    switch (R) {
        case 1:
            if constexpr (EPI != EPI_LOGITS) return gemv_launch_ks<Q8, SM, 1, EPI>(KS, grid, a, KC, lds, st);
            break;
        case 2: return gemv_launch_ks<Q8, SM, 2, EPI>(KS, grid, a, KC, lds, st);
        case 4:
            if constexpr (SM == 1 && (EPI == EPI_STORE || EPI == EPI_LOGITS))
                return gemv_launch_ks<Q8, SM, 4, EPI>(KS, grid, a, KC, lds, st);
            break;
    }
    return hipErrorInvalidValue;
}

template <int Q8, int EPI>
hipError_t gemv_dispatch(const GemvArgs &a, hipStream_t st) {
    constexpr int E = Q8 ? 16 : 8;
    const int slices = a.K / (64 * E);  // 16-byte slices per lane per row over the whole K
    // Slices per chunk: one vector keeps up to four slices per lane per row in registers (the whole row
    // span for K <= 4*64*E); several vectors stage at most 64 KB of inputs in LDS per chunk.
    int KS;
    if (a.S == 1) {
        KS = (slices <= 4 || (!Q8 && slices == 6)) ? slices
                                                  : (slices % 4 == 0 ? 4 : slices % 3 == 0 ? 3 : slices % 2 == 0 ? 2 : 1);
    } else {
        KS = slices % 2 == 0 ? 2 : 1;
        while (KS > 1 && (size_t)a.S * KS * 64 * E > 16384) KS /= 2;
    }
    int R;
    if (a.S == 1) {
        R = EPI == EPI_LOGITS ? 4 : EPI == EPI_STORE ? 2 : 1;
        if (EPI == EPI_STORE && (a.N + 2 * 4 - 1) / (2 * 4) < 256) R = 1;
    } else {
        R = (EPI == EPI_LOGITS || (EPI != EPI_SWIGLU && (a.N + 7) / 8 >= 256)) ? 2 : 1;
    }
    while (KS >= 4 && R > 2) R /= 2;
    if (EPI == EPI_LOGITS && R < 2) R = 2;
    const int KC = KS * 64 * E;
    const bool single = KC >= a.K;
    const size_t lds = (size_t)a.S * KC * sizeof(float);
    const int n_groups = (a.N + R - 1) / R;
    int grid = (n_groups + 3) / 4;
    if (single && EPI == EPI_LOGITS && grid > 1024) grid = 1024;  // waves walk several groups
    if (EPI == EPI_LOGITS && grid > kLmMaxBlocks) return hipErrorInvalidValue;
    hipError_t e = a.S == 1 ? gemv_launch_r<Q8, 1, EPI>(R, KS, grid, a, KC, lds, st)
                            : gemv_launch_r<Q8, kMaxSeq, EPI>(R, KS, grid, a, KC, lds, st);
    if (e != hipSuccess || EPI != EPI_LOGITS) return e;
    hipLaunchKernelGGL(argmax_finalize_kernel, dim3(a.S), dim3(256), 0, st, a.argpart, grid, a.S, a.argmax_out, a.len,
                       a.commit_add, (const int *)a.status);
    return hipGetLastError();
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
// and written as the split's partial (running max, running sum, unnormalised output); attn_merge_kernel
// combines the splits.
// ---------------------------------------------------------------------------------------------------
// K/V of the newly appended position as 8 packed bf16 pairs (the LDS copy holds the bf16 bits per dim).
__device__ __forceinline__ void new_kv_from_lds(const float *knew, const float *vnew, int dsub, uint4 &k, uint4 &v) {
    uint32_t kw[4], vw[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        kw[q] = __float_as_uint(knew[dsub + 2 * q]) | (__float_as_uint(knew[dsub + 2 * q + 1]) << 16);
        vw[q] = __float_as_uint(vnew[dsub + 2 * q]) | (__float_as_uint(vnew[dsub + 2 * q + 1]) << 16);
    }
    k = make_uint4(kw[0], kw[1], kw[2], kw[3]);
    v = make_uint4(vw[0], vw[1], vw[2], vw[3]);
}

template <int G>
__global__ __launch_bounds__(256) void attn_decode_kernel(AttnDecodeArgs a) {
    const int split = blockIdx.x, kvh = blockIdx.y, s = blockIdx.z;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    __shared__ float qs[G][kHeadDim];
    __shared__ float knew[kHeadDim], vnew[kHeadDim];
    __shared__ float red[4];
    __shared__ float wm[4][G], wl[4][G];
    __shared__ float wacc[4][G][kHeadDim];

    const int pos = a.len[s];
    const int n = pos + 1;
    int chunk = (n + a.n_split - 1) / a.n_split;
    chunk = (chunk + 15) & ~15;
    const int start = split * chunk;
    const int end = min(n, start + chunk);
    const size_t head_off = (size_t)s * a.seq_stride + (size_t)kvh * a.max_ctx * kHeadDim;
    const uint16_t *kb = a.kcache + head_off;
    const uint16_t *vb = a.vcache + head_off;
    const int dsub = (lane & 15) * 8;
    const int prow = lane >> 4;

    // K/V of this wave's first 16-position group, issued before the query prologue.  The new position is
    // excluded here: it is written below and read in the loop after the append.
    uint4 kr[4], vr[4];
    bool val[4];
    int j0 = start + 16 * wave;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int p = j0 + 4 * i + prow;
        val[i] = p < end;
        if (val[i] && p != pos) {
            kr[i] = load_nt16(kb + (size_t)p * kHeadDim + dsub);
            vr[i] = load_nt16(vb + (size_t)p * kHeadDim + dsub);
        } else {
            kr[i] = make_uint4(0, 0, 0, 0);
            vr[i] = make_uint4(0, 0, 0, 0);
        }
    }

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

    // ---- append the new key/value (only the workgroup whose split holds the new position)
    const bool owner = pos >= start && pos < end;
    if (owner) {
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
        const uint16_t b = f32_to_bf16(out);
        *((uint16_t *)(is_k ? kb : vb) + (size_t)pos * kHeadDim + d) = b;
        __syncthreads();  // every lane has read knew for its rotation
        (is_k ? knew : vnew)[d] = __uint_as_float((uint32_t)b);
        __syncthreads();
        // the new position is taken from LDS (its global store may still be in flight)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (j0 + 4 * i + prow == pos) new_kv_from_lds(knew, vnew, dsub, kr[i], vr[i]);
    }

    // ---- stream this split's positions
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

    while (j0 < end) {
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
                d = row16_sum(d);  // the 16 lanes of a row hold one position's dims (DPP, no LDS round trip)
                sc[h][i] = val[i] ? d * sl2 : -INFINITY;
            }
        }
        float vf[4][8];
#pragma unroll
        for (int i = 0; i < 4; ++i) unpack_bf16x8(vr[i], vf[i]);
        // next group's loads go out before this group's softmax and V accumulation
        j0 += 64;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int p = j0 + 4 * i + prow;
            val[i] = p < end;
            if (val[i] && p != pos) {
                kr[i] = load_nt16(kb + (size_t)p * kHeadDim + dsub);
                vr[i] = load_nt16(vb + (size_t)p * kHeadDim + dsub);
            } else if (val[i]) {
                new_kv_from_lds(knew, vnew, dsub, kr[i], vr[i]);
            } else {
                kr[i] = make_uint4(0, 0, 0, 0);
                vr[i] = make_uint4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float tm = fmaxf(fmaxf(sc[h][0], sc[h][1]), fmaxf(sc[h][2], sc[h][3]));  // uniform within a row
            tm = fmaxf(fmaxf(lane_get(tm, 0), lane_get(tm, 16)), fmaxf(lane_get(tm, 32), lane_get(tm, 48)));
            const float mn = fmaxf(m[h], tm);
            const float alpha = __builtin_amdgcn_exp2f(m[h] - mn);  // v_exp_f32 (exactly 0 at -inf)
            l[h] *= alpha;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] *= alpha;
            m[h] = mn;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p = __builtin_amdgcn_exp2f(sc[h][i] - mn);
                l[h] += p;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[h][e] += p * vf[i][e];
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
}

// Merge of one (sequence, query head)'s context splits, in split order (the result does not depend on
// which split finished first): M = max m_s, f_s = 2^(m_s - M) / sum_s 2^(m_s - M) l_s, o = sum_s f_s o_s.
// Grid (HQ, S), one thread per head dimension.  Runs as its own kernel: the partials of every split are
// visible after the attention kernel's boundary, which is cheaper on this chip than an in-kernel arrival
// ticket (device-coherent stores, their completion and an atomic).
__global__ __launch_bounds__(kHeadDim) void attn_merge_kernel(const float *part, int HQ, int n_split, float *out,
                                                              int ldo, uint16_t *o_hi, uint16_t *o_lo) {
    static_assert(kMaxSplit == 64, "one split per lane of a wave");
    __shared__ float fm[kMaxSplit], fl[kMaxSplit];
    const int h = blockIdx.x, s = blockIdx.y, d = threadIdx.x;
    const float *p0 = part + (((size_t)s * HQ + h) * kMaxSplit) * kPartStride;
    float ov[kMaxSplit];
#pragma unroll
    for (int sp = 0; sp < kMaxSplit; ++sp) ov[sp] = sp < n_split ? p0[sp * kPartStride + 2 + d] : 0.f;
    if (d < kMaxSplit) {
        fm[d] = d < n_split ? p0[d * kPartStride] : -INFINITY;
        fl[d] = d < n_split ? p0[d * kPartStride + 1] : 0.f;
    }
    __syncthreads();
    if (d < 64) {
        const float mv = fm[d];
        const float M = wave_max(mv);
        const float f = mv == -INFINITY ? 0.f : exp2f(mv - M);
        const float L = wave_sum(f * fl[d]);
        fm[d] = f / L;
    }
    __syncthreads();
    float o = 0.f;
#pragma unroll
    for (int sp = 0; sp < kMaxSplit; ++sp) o += fm[sp] * ov[sp];
    out[(size_t)s * ldo + h * kHeadDim + d] = o;
    if (o_hi) {  // o_proj operand of the batched Q8 path: f16 high part and remainder
        const _Float16 hv = (_Float16)o;
        const size_t i = mfma_opnd_index(h * kHeadDim + d, s);
        o_hi[i] = __builtin_bit_cast(uint16_t, hv);
        o_lo[i] = __builtin_bit_cast(uint16_t, (_Float16)(o - (float)hv));
    }
}

// Embedding: x[s] = row tokens[s] of the table, widened (bf16) or dequantised (code * scale).
template <int Q8>
__global__ void embed_kernel(const void *table, const float *scales, int H, const int *tokens, float *x,
                             int *status, int vocab) {
    const int s = blockIdx.y;
    const int k = blockIdx.x * blockDim.x + threadIdx.x;
    int tok = tokens[s];
    if (tok < 0 || tok >= vocab) {
        if (k == 0) atomicOr(status, kStatusBadToken);
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

__global__ void set_lens_kernel(int *len, int n, LenVals vals, int mask, int *status, int clear_status,
                                uint32_t *epoch) {
    const int t = threadIdx.x;
    if (t < n && (mask >> t) & 1) len[t] = vals.v[t];
    if (t == 0 && clear_status) {
        *status = 0;
        // a launch of the single-launch decode that gave up did not advance the tag base: move it past any
        // word that launch may have written
        *epoch += 1u << 20;
    }
}

// Commit of positions appended without a logits step (earlier prefill chunks, hidden-state steps); like the
// final commit, nothing is committed once the status word holds a failure.
__global__ void commit_kernel(int *len, int n, int add, const int *status) {
    const int t = threadIdx.x;
    if (t < n && *status == 0) len[t] += add;
}

template <int Q8>
__global__ void dequant_kernel(const void *w, const float *scales, long long total, int cols, float *out) {
    (void)cols;  // rows are whole 32-blocks (cols % 32 == 0), so element i's block is i / 32
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total) return;
    if (Q8)
        out[i] = (float)((const int8_t *)w)[i] * scales[i >> 5];
    else
        out[i] = bf16_to_f32(((const uint16_t *)w)[i]);
}

}  // namespace

hipError_t launch_argmax_finalize(const float *argpart, int nparts, int S, int *argmax_out, int *len, int commit_add,
                                  const int *status, hipStream_t st) {
    hipLaunchKernelGGL(argmax_finalize_kernel, dim3(S), dim3(256), 0, st, argpart, nparts, S, argmax_out, len,
                       commit_add, status);
    return hipGetLastError();
}

hipError_t launch_gemv(bool q8, GemvEpi epi, const GemvArgs &a, hipStream_t st) {
    if (a.mfma) return q8 ? launch_gemv_mfma(epi, a, st) : hipErrorInvalidValue;
    if (a.S < 1 || a.S > kMaxSeq || a.K % (q8 ? 1024 : 512)) return hipErrorInvalidValue;
#define QW3_GEMV_EPI(Q)                                                     \
    switch (epi) {                                                          \
        case EPI_STORE: return gemv_dispatch<Q, EPI_STORE>(a, st);          \
        case EPI_RESID: return gemv_dispatch<Q, EPI_RESID>(a, st);          \
        case EPI_SWIGLU: return gemv_dispatch<Q, EPI_SWIGLU>(a, st);        \
        case EPI_LOGITS: return gemv_dispatch<Q, EPI_LOGITS>(a, st);        \
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
    hipLaunchKernelGGL(attn_merge_kernel, dim3(a.HQ, a.S), dim3(kHeadDim), 0, st, a.part, a.HQ, a.n_split, a.out,
                       a.ldo, a.o_hi, a.o_lo);
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
                           uint32_t *epoch, hipStream_t st) {
    LenVals v{};
    for (int i = 0; i < n && i < kMaxSeq; ++i) v.v[i] = vals[i];
    hipLaunchKernelGGL(set_lens_kernel, dim3(1), dim3(64), 0, st, len_dev, n, v, mask, status, clear_status, epoch);
    return hipGetLastError();
}

hipError_t launch_commit(int *len_dev, int n, int add, const int *status, hipStream_t st) {
    hipLaunchKernelGGL(commit_kernel, dim3(1), dim3(64), 0, st, len_dev, n, add, status);
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
