// Persistent single-launch decode of one token of one sequence for gfx950 (hidden size 1024, head_dim 128).
//
// One launch runs the whole layer stack of [P1] section 5 ("Transformer Layer Execution Loop") for one token:
// 256 workgroups stay resident and walk six dependent phases per layer,
//   Q  RMSNorm + Q/K/V rows                 ([P1] section 2 items 1-2)
//   A  QK-Norm, RoPE, KV append, attention   (items 3-5; one workgroup per (KV head, context split))
//   M  merge of the context splits           (item 5, exact online-softmax combination)
//   O  o_proj + residual                     (item 6)
//   U  RMSNorm + gate/up + SwiGLU            (items 6-7)
//   D  down + residual                       (item 7)
// Every phase is spread over all 1024 waves of the grid; phase outputs travel between workgroups as 8-byte
// words (f32 value, 32-bit epoch tag) written and polled with device-coherent relaxed atomics, so a consumer
// needs no separate flag: a word is ready when its tag equals the tag of (layer, phase) in this launch.
// While a workgroup waits for a phase's inputs, that phase's weights (and, for attention, the cached K/V of
// the old positions) are already in flight into registers: weight streaming from HBM overlaps the exchange
// latency instead of following it.  Hidden row r (r < 1024) is owned by global wave r in the o_proj and down
// phases, which keeps the residual stream of that row in a register.
//
// Every wait is bounded (a fixed number of polling rounds, tens of milliseconds).  A workgroup that times out sets bit 4 of
// the status word; every poll also watches that bit, so the whole grid leaves promptly and the status word
// reports a device error instead of a hang.
//
// Page titles used in citations:
//   [P1] "Scalar-Native Qwen3 Reference Runtime As The Numerical Authority"
//   [P4] "Portable WebAssembly Runtime Architecture for TinyRustLM"
#include <math.h>

#include "common.h"

namespace qw3 {

namespace {

constexpr int kWaves = kMegaWaves;
constexpr int kNW = kMegaGrid * kWaves;  // waves in the grid
constexpr int kHid = 1024;               // hidden size of this kernel (= kNW: one owned row per wave)
// Poll bound: rounds of device-coherent loads (each at least one memory round trip, well over 0.25 us), so
// 2^18 rounds outlast 50 ms while a legitimate wait lasts microseconds.
constexpr int kPollRounds = 1 << 18;
constexpr int kMegaBuf = 3072;  // floats per LDS input buffer (largest phase input: intermediate <= 3072)
// Quads (4 positions) per attention chunk.  With G <= 2 query heads per KV head a pass covers 20 positions per
// wave, so up to 2560 cached positions (128 wave slots) take a single online-softmax pass in every wave, and
// past 2048 no wave needs a second pass for the one quad left over from an even share of four.  Four query heads
// per KV head keep chunks of four quads (registers).
template <int G>
constexpr int chunk_quads() { return G <= 2 ? 5 : 4; }

static_assert(kHid == kNW, "one hidden row per wave");

// LDS layout of the vectors the dot products read as lane-contiguous 16-element slices (64-byte lane stride):
// four floats of padding after every 32 elements, so the 16-byte reads of the eight lanes served together fall
// in different banks (without it the decode kernel's LDS counters showed bank conflicts in 54 % of its active
// LDS cycles; the layer stack is 6 us per token faster with it).  Slices of 8 or 16 elements never straddle a
// padding gap.  The polls of the hidden vector, the attention output and the SwiGLU activations write this
// layout; the attention and merge inputs stay dense.
constexpr int kPadShift = 5;
__device__ __forceinline__ int padx(int i) { return i + ((i >> kPadShift) << 2); }
constexpr int padded(int n) { return n + ((n >> kPadShift) << 2); }

// Phase timing (diagnostic builds only, -DQW3_MEGA_STAMPS): thread 0 of every workgroup records the 100 MHz
// s_memrealtime clock when a phase's inputs have all arrived (k = 0) and when it has published its outputs
// (k = 1), per (layer, phase); qw3_mega_stamps copies the table out.  The clock is global to the device, so
// stamps of different workgroups compare directly.
#ifdef QW3_MEGA_STAMPS
constexpr int kStampLayers = 64;
__device__ uint64_t g_mega_stamps[kStampLayers * 6 * 2 * kMegaGrid + kMegaGrid];
#define QW3_STAMP(l, ph, k)                                                                                   \
    do {                                                                                                      \
        if (threadIdx.x == 0 && (l) < kStampLayers)                                                           \
            __builtin_nontemporal_store((uint64_t)__builtin_amdgcn_s_memrealtime(),                            \
                                        &g_mega_stamps[(((l) * 6 + (ph)) * 2 + (k)) * kMegaGrid + blockIdx.x]); \
    } while (0)
#else
#define QW3_STAMP(l, ph, k) \
    do {                    \
    } while (0)
#endif

__device__ __forceinline__ void put(uint64_t *p, float v, uint32_t tag) {
    __hip_atomic_store(p, ((uint64_t)tag << 32) | (uint64_t)__float_as_uint(v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t get(const uint64_t *p) {
    return __hip_atomic_load((uint64_t *)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool timed_out(int *status) {
    return (__hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & kStatusTimeout) != 0;
}

__device__ __forceinline__ void unpack_i8x16(const uint4 &w, float (&o)[16]) {
    const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int b = 0; b < 4; ++b) o[4 * j + b] = (float)(int8_t)(d[j] >> (8 * b));
}
__device__ __forceinline__ void unpack_bf16x8(const uint4 &w, float (&o)[8]) {
    const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        o[2 * j] = bf16_lo(d[j]);
        o[2 * j + 1] = bf16_hi(d[j]);
    }
}

// Waits until the n tagged words src(i), i < n, all carry `tag` and writes their values to dst[i] (LDS).
// Thread t polls words t, t + 256, ...; words already seen are not loaded again.  Starts with a workgroup
// barrier, so earlier readers of dst have finished.  Returns false on timeout or when another workgroup has
// reported one.
template <int NPT, bool PAD = false, typename Addr>
__device__ __forceinline__ bool poll(Addr src, int n, uint32_t tag, float *dst, int *status) {
    const int tid = threadIdx.x;
    uint32_t pending = 0;
#pragma unroll
    for (int j = 0; j < NPT; ++j)
        if (tid + 256 * j < n) pending |= 1u << j;
    __syncthreads();  // earlier readers of dst are done
    for (int round = 0; pending; ++round) {
        uint64_t v[NPT];
#pragma unroll
        for (int j = 0; j < NPT; ++j)
            if ((pending >> j) & 1u) v[j] = get(src(tid + 256 * j));
#pragma unroll
        for (int j = 0; j < NPT; ++j) {
            if (((pending >> j) & 1u) && (uint32_t)(v[j] >> 32) == tag) {
                dst[PAD ? padx(tid + 256 * j) : tid + 256 * j] = __uint_as_float((uint32_t)v[j]);
                pending &= ~(1u << j);
            }
        }
        // another workgroup's timeout is checked now and then; this one's after the round bound
        if (pending && (round >= kPollRounds || ((round & 31) == 31 && timed_out(status)))) return false;
    }
    return true;
}

// Workgroup-wide agreement after a poll: true when every thread's poll succeeded.
__device__ __forceinline__ bool all_ok(bool ok, int &s_fail, int *status) {
    // workgroup-scope atomics on the LDS flag (no generic-pointer volatile access, which would wait for every
    // global memory operation in flight)
    if (!ok) __hip_atomic_store(&s_fail, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    __syncthreads();
    if (__hip_atomic_load(&s_fail, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) {
        if (threadIdx.x == 0) atomicOr(status, kStatusTimeout);
        return false;
    }
    return true;
}

// Weight rows -> registers.  Lane `lane` holds, for chunk c of a row, the 16-byte slice starting at element
// c*64*E + lane*E (E = 16 int8 codes or 8 bf16 values), and for Q8 the scale of that slice's 32-block.
// Every slot is loaded, unconditionally: slots of absent rows or chunks read row 0 / chunk 0 and are never
// used.  A fixed number of loads per call lets the compiler wait for exactly the loads a computation needs
// (the vector memory counter drains in issue order), instead of for everything in flight.
template <int Q8, int R, int C>
__device__ __forceinline__ void load_rows(const uint8_t *w, const float *s, int K, const int (&row)[R],
                                          const bool (&rv)[R], int nch, int lane, uint4 (&wv)[R][C],
                                          float (&sc)[R][C]) {
    constexpr int E = Q8 ? 16 : 8;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const size_t rr = rv[r] ? (size_t)row[r] : 0;
            const int k = (c < nch ? c : 0) * 64 * E + lane * E;
            wv[r][c] = load_nt16(w + (rr * K + k) * (Q8 ? 1 : 2));
            if constexpr (Q8) sc[r][c] = s[rr * (K / 32) + (k >> 5)];
            else sc[r][c] = 0.f;
        }
}

// Lane's share of one row's dot product with the input vector xl (LDS), chunks c < nch.
template <int Q8, int C>
__device__ __forceinline__ float dot_lds(const uint4 (&wv)[C], const float (&sc)[C], const float *xl, int nch,
                                         int lane) {
    constexpr int E = Q8 ? 16 : 8;
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < C; ++c) {
        if (c < nch) {
            const float4 *xp = (const float4 *)(xl + padx(c * 64 * E + lane * E));
            float xv[E];
#pragma unroll
            for (int q = 0; q < E / 4; ++q) {
                const float4 v = xp[q];
                xv[4 * q] = v.x;
                xv[4 * q + 1] = v.y;
                xv[4 * q + 2] = v.z;
                xv[4 * q + 3] = v.w;
            }
            if constexpr (Q8) {
                float wf[16];
                unpack_i8x16(wv[c], wf);
                float d = 0.f;
#pragma unroll
                for (int e = 0; e < 16; ++e) d += wf[e] * xv[e];
                acc += d * sc[c];
            } else {
                float wf[8];
                unpack_bf16x8(wv[c], wf);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc += wf[e] * xv[e];
            }
        }
    }
    return acc;
}

// Lane's share of a row's dot product with inputs held in registers (K = 1024: CH chunks of E values).
template <int Q8, int CH>
__device__ __forceinline__ float dot_reg(const uint4 (&wv)[CH], const float (&sc)[CH], const float (&xr)[CH][Q8 ? 16 : 8]) {
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        if constexpr (Q8) {
            float wf[16];
            unpack_i8x16(wv[c], wf);
            float d = 0.f;
#pragma unroll
            for (int e = 0; e < 16; ++e) d += wf[e] * xr[c][e];
            acc += d * sc[c];
        } else {
            float wf[8];
            unpack_bf16x8(wv[c], wf);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc += wf[e] * xr[c][e];
        }
    }
    return acc;
}

// Lane's slice of a 1024-long f32 vector (the elements that lane's weight chunks multiply).
template <int Q8, int CH>
__device__ __forceinline__ void load_slice(const float *v, int lane, float (&out)[CH][Q8 ? 16 : 8]) {
    constexpr int E = Q8 ? 16 : 8;
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
        for (int q = 0; q < E / 4; ++q) {
            const float4 t = *(const float4 *)(v + c * 64 * E + lane * E + 4 * q);
            out[c][4 * q] = t.x;
            out[c][4 * q + 1] = t.y;
            out[c][4 * q + 2] = t.z;
            out[c][4 * q + 3] = t.w;
        }
}

// RMSNorm of the 1024-vector xs (LDS) with weight slice w ([P1] section 2 items 1 and 6: w * (x / sqrt(mean(x^2)
// + eps))), returning the lane's slice in registers.  Every wave reduces the whole vector itself, from the
// same 16-byte LDS reads that fetch its slice (the slices of the 64 lanes tile the vector); 1/sqrt is one
// v_rsq_f32 (within 1 ulp of the correctly rounded quotient, well inside the decode's tolerance).
template <int Q8, int CH>
__device__ __forceinline__ void rms_slice(const float *xs, const float (&w)[CH][Q8 ? 16 : 8], float eps, int lane,
                                          float (&xr)[CH][Q8 ? 16 : 8]) {
    constexpr int E = Q8 ? 16 : 8;
    static_assert(CH * 64 * E == kHid, "the lane slices cover the vector once");
    float xv[CH][E];
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
        for (int q = 0; q < E / 4; ++q) {
            const float4 t = *(const float4 *)(xs + padx(c * 64 * E + lane * E) + 4 * q);
            xv[c][4 * q] = t.x;
            xv[c][4 * q + 1] = t.y;
            xv[c][4 * q + 2] = t.z;
            xv[c][4 * q + 3] = t.w;
        }
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
        for (int e = 0; e < E; ++e) ss += xv[c][e] * xv[c][e];
    ss = wave_sum_fast(ss);
    const float inv = __builtin_amdgcn_rsqf(ss / (float)kHid + eps);
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
        for (int e = 0; e < E; ++e) xr[c][e] = w[c][e] * (xv[c][e] * inv);
}

// ---- q8 x q8 products (weight mode 2): activations quantized to int8 per 32-block on the fly ([P3] section 5
// "Q8_0 Mixed-Precision Matrix Multiplication") -------------------------------------------------------------
// The block scale is d = max|x| / 127 over the block's 32 inputs, each code rounds x / d to nearest (ties away
// from zero) and is clamped to [-127, 127].  A NaN in the block makes d NaN; a block whose d is zero or not
// finite gets zero codes, so a non-finite input reaches the products through d instead of being repaired.

// One lane's 16 products of int8 weight codes and activation codes summed in int32 (at most 16 * 127 * 127),
// converted to f32 and scaled by both block scales.
__device__ __forceinline__ float dot16_a8(const uint4 &w, const uint32_t (&q)[4], float sw, float da) {
    int acc = __builtin_amdgcn_sdot4((int)w.x, (int)q[0], 0, false);
    acc = __builtin_amdgcn_sdot4((int)w.y, (int)q[1], acc, false);
    acc = __builtin_amdgcn_sdot4((int)w.z, (int)q[2], acc, false);
    acc = __builtin_amdgcn_sdot4((int)w.w, (int)q[3], acc, false);
    return (float)acc * (sw * da);
}

// The workgroup quantizes an n-element input (n a multiple of 1024) once, for all four waves: in each pass of
// 1024 elements thread t takes elements 4t..4t+3, so a 32-block spans eight lanes of a row, whose max (and NaN
// flag) three DPP steps share.  With NORM the elements are the RMSNorm outputs nw * (x * inv) of the pass, else
// x itself.  Writes codes[k / 4] = the int8 codes of elements k..k+3 (lowest element in the lowest byte) and
// dsc[k / 32] = the block scale.
template <bool NORM>
__device__ __forceinline__ void quant_wg(const float *x, int n, const float4 &nw, float inv, uint32_t *codes,
                                         float *dsc) {
    const int t = threadIdx.x;
    for (int base = 0; base < n; base += 1024) {
        const float4 r = *(const float4 *)(x + padx(base + 4 * t));
        float v[4] = {r.x, r.y, r.z, r.w};
        if constexpr (NORM) {
            v[0] = nw.x * (v[0] * inv);
            v[1] = nw.y * (v[1] * inv);
            v[2] = nw.z * (v[2] * inv);
            v[3] = nw.w * (v[3] * inv);
        }
        float m = 0.f, nan = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float a = fabsf(v[e]);
            nan = a != a ? 1.f : nan;
            m = fmaxf(m, a);
        }
        m = fmaxf(m, dpp_mov<0xB1>(m));   // quad_perm [1,0,3,2]
        m = fmaxf(m, dpp_mov<0x4E>(m));   // quad_perm [2,3,0,1]
        m = fmaxf(m, dpp_mov<0x141>(m));  // row_half_mirror: the other quad of the eight lanes
        nan = fmaxf(nan, dpp_mov<0xB1>(nan));
        nan = fmaxf(nan, dpp_mov<0x4E>(nan));
        nan = fmaxf(nan, dpp_mov<0x141>(nan));
        const float d = nan != 0.f ? __builtin_nanf("") : m / 127.0f;
        const bool ok = d > 0.f && d < INFINITY;
        uint32_t w = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const float c = ok ? fminf(fmaxf(roundf(v[b] / d), -127.f), 127.f) : 0.f;
            w |= ((uint32_t)(int)c & 0xffu) << (8 * b);
        }
        codes[(base >> 2) + t] = w;
        if ((t & 7) == 0) dsc[(base >> 5) + (t >> 3)] = d;
    }
}

// Lane's share of a q8 x q8 row product with the codes quant_wg left in LDS: chunk c holds elements
// c*1024 + lane*16 .. +16, one 16-byte code read and the scale of their block.
template <int C>
__device__ __forceinline__ float dot_codes(const uint4 (&wv)[C], const float (&sc)[C], const uint32_t *codes,
                                           const float *dsc, int nch, int lane) {
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < C; ++c) {
        if (c < nch) {
            const uint4 q4 = *(const uint4 *)(codes + c * 256 + lane * 4);
            const uint32_t q[4] = {q4.x, q4.y, q4.z, q4.w};
            acc += dot16_a8(wv[c], q, sc[c], dsc[c * 32 + (lane >> 1)]);
        }
    }
    return acc;
}

// 1 / sqrt(mean(x^2) + eps) of the 1024-vector xs (LDS), the factor rms_slice applies, in every lane.
__device__ __forceinline__ float rms_inv(const float *xs, float eps, int lane) {
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < kHid / 64; ++k) {
        const float v = xs[padx(lane + 64 * k)];
        ss += v * v;
    }
    ss = wave_sum_fast(ss);
    return 1.0f / sqrtf(ss / (float)kHid + eps);
}

// Cached K/V of one chunk of CQ 4-position quads for this lane: positions 4*(q0 + i) + lane/16, dims
// (lane%16)*8..+8.  Always 2 * CQ loads: slots of quads at or after qe, or of positions at or after `pos`
// (the new position is written in this launch and taken from LDS), read position 0 and are never used.
template <int CQ>
__device__ __forceinline__ void load_chunk(const uint16_t *kb, const uint16_t *vb, int q0, int qe, int pos,
                                           int lane, uint4 (&kr)[CQ], uint4 (&vr)[CQ]) {
    const int dsub = (lane & 15) * 8, prow = lane >> 4;
#pragma unroll
    for (int i = 0; i < CQ; ++i) {
        const int p = 4 * (q0 + i) + prow;
        const size_t pc = (q0 + i < qe && p < pos) ? (size_t)p : 0;
        kr[i] = load_nt16(kb + pc * kHeadDim + dsub);
        vr[i] = load_nt16(vb + pc * kHeadDim + dsub);
    }
}

// 2^x on the transcendental unit (one v_exp_f32; exactly 0 at -inf).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Online-softmax update with one chunk of cached positions: NQ quads (1..5) starting at quad q0 ([P1] section 2
// item 5; running max m, running sum l, unnormalised accumulator acc; each lane row keeps its own l and acc).
// Scores are in log2 units (the scale sl2 carries log2(e)), so every exponential is a single 2^x.
template <int G, int NQ, int CQ>
__device__ __forceinline__ void attend_chunk(uint4 (&kr)[CQ], uint4 (&vr)[CQ], int q0, int pos, int lane,
                                             const float (&qr)[G][8], float sl2, float (&m)[G], float (&l)[G],
                                             float (&acc)[G][8]) {
    const int prow = lane >> 4;
    bool val[NQ];
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
        val[i] = 4 * (q0 + i) + prow < pos;
        if (!val[i]) {  // placeholder slot: keep stale cache bits out of the sums
            kr[i] = make_uint4(0, 0, 0, 0);
            vr[i] = make_uint4(0, 0, 0, 0);
        }
    }
    float sc[G][NQ];
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
        float kf[8];
        unpack_bf16x8(kr[i], kf);
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float d = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) d += qr[h][e] * kf[e];
            d = row16_sum(d);  // the 16 lanes of a row hold one position's dims
            sc[h][i] = val[i] ? d * sl2 : -INFINITY;
        }
    }
    float vf[NQ][8];
#pragma unroll
    for (int i = 0; i < NQ; ++i) unpack_bf16x8(vr[i], vf[i]);
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float tm = sc[h][0];  // uniform within a row
#pragma unroll
        for (int i = 1; i < NQ; ++i) tm = fmaxf(tm, sc[h][i]);
        tm = fmaxf(fmaxf(lane_get(tm, 0), lane_get(tm, 16)), fmaxf(lane_get(tm, 32), lane_get(tm, 48)));
        const float mn = fmaxf(m[h], tm);
        if (mn == -INFINITY) continue;  // nothing valid yet in this lane row set
        const float alpha = exp2_hw(m[h] - mn);
        l[h] *= alpha;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] *= alpha;
        m[h] = mn;
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            const float p = exp2_hw(sc[h][i] - mn);
            l[h] += p;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] += p * vf[i][e];
        }
    }
}

// attend_chunk for a run of nq quads (the same in every lane): full chunks take the CQ-quad form, the last
// chunk of a run its own length
template <int G, int CQ>
__device__ __forceinline__ void attend_run(uint4 (&kr)[CQ], uint4 (&vr)[CQ], int q0, int nq, int pos, int lane,
                                           const float (&qr)[G][8], float sl2, float (&m)[G], float (&l)[G],
                                           float (&acc)[G][8]) {
    static_assert(CQ == 4 || CQ == 5, "chunks of four or five quads");
    if (nq >= CQ) attend_chunk<G, CQ, CQ>(kr, vr, q0, pos, lane, qr, sl2, m, l, acc);
    else if (CQ == 5 && nq == 4) attend_chunk<G, 4, CQ>(kr, vr, q0, pos, lane, qr, sl2, m, l, acc);
    else if (nq == 3) attend_chunk<G, 3, CQ>(kr, vr, q0, pos, lane, qr, sl2, m, l, acc);
    else if (nq == 2) attend_chunk<G, 2, CQ>(kr, vr, q0, pos, lane, qr, sl2, m, l, acc);
    else if (nq == 1) attend_chunk<G, 1, CQ>(kr, vr, q0, pos, lane, qr, sl2, m, l, acc);
}

// Online-softmax update with the new position (key kn, value vn in LDS, already rounded to bf16); lane row 0
// carries its weight.
template <int G>
__device__ __forceinline__ void attend_new(const float *kn, const float *vn, int lane, const float (&qr)[G][8],
                                           float sl2, float (&m)[G], float (&l)[G], float (&acc)[G][8]) {
    const int dsub = (lane & 15) * 8;
    // the lane's eight dims of the new key and value, read once (unconditional 16-byte LDS reads)
    float kf[8], vf[8];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const float4 k4 = *(const float4 *)(kn + dsub + 4 * q), v4 = *(const float4 *)(vn + dsub + 4 * q);
        kf[4 * q] = k4.x, kf[4 * q + 1] = k4.y, kf[4 * q + 2] = k4.z, kf[4 * q + 3] = k4.w;
        vf[4 * q] = v4.x, vf[4 * q + 1] = v4.y, vf[4 * q + 2] = v4.z, vf[4 * q + 3] = v4.w;
    }
    const float row0 = lane < 16 ? 1.f : 0.f;
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) d += qr[h][e] * kf[e];
        const float sc = row16_sum(d) * sl2;  // every row computes the same full dot product
        const float mn = fmaxf(m[h], sc);
        const float alpha = exp2_hw(m[h] - mn), pw = exp2_hw(sc - mn) * row0;
        l[h] = l[h] * alpha + pw;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = acc[h][e] * alpha + pw * vf[e];
        m[h] = mn;
    }
}

}  // namespace

template <int Q8, int G>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void decode_mega_kernel(MegaArgs a) {
    constexpr int E = Q8 ? 16 : 8;
    constexpr int CH = kHid / (64 * E);  // chunks per lane of a 1024-long row
    constexpr int KO_MAX = Q8 ? 2 : 4;   // q_dim <= 2048
    constexpr int KD_MAX = Q8 ? 3 : 6;   // intermediate <= 3072
    constexpr int RQ_MAX = 4;            // Q/K/V rows per wave (<= 4096 rows)
    constexpr int RU_MAX = 3;            // gate/up units per wave (<= 3072 units)
    static_assert(kXwReps <= 32, "one lane of a half wave per copy of a published word");
    constexpr int PW = 2 + kHeadDim;     // words of one attention partial (max, sum, o[128])

    __shared__ __attribute__((aligned(16))) float xs[padded(kHid)];
    __shared__ __attribute__((aligned(16))) float big[4096];
    static_assert(padded(kMegaBuf) <= 4096, "padded phase inputs fit the buffer");
    __shared__ __attribute__((aligned(16))) float wacc[kWaves * G * kHeadDim];  // [wave][G][128]
    __shared__ float wm[kWaves][G], wl[kWaves][G];
    __shared__ int s_fail;
    // q8 x q8 (Q8 == 2): the workgroup's int8 codes and block scales of the current phase input
    __shared__ __attribute__((aligned(16))) uint32_t qcode[kMegaBuf / 4];
    __shared__ float qdsc[kMegaBuf / 32];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int b = blockIdx.x;
    const int gw = b * kWaves + wave;  // global wave id = owned hidden row
    const int HQ = a.HQ, HKV = a.HKV, I = a.I;
    const int q_dim = HQ * kHeadDim, kv_dim = HKV * kHeadDim, Nqkv = q_dim + 2 * kv_dim;
    const int KO = q_dim / (64 * E), KD = I / (64 * E);
    const int SP = kMegaGrid / HKV;  // context splits per KV head
    const uint32_t ep = a.epoch[0];
    const int pos = a.len[0];
    if (tid == 0) s_fail = 0;

    // this workgroup's attention share: KV head g, split sp.  The cached positions [0, pos) form quads of four;
    // wave slot ws = 4 sp + wave takes a contiguous run of quads [qa, qe), floor(quads / nslot) of them plus one
    // for the first quads % nslot slots, so no wave holds more than one quad beyond the others.  The runs are
    // processed chunk_quads<G>() quads (20 or 16 positions) at a time.  The new position goes to the last slot, which never holds
    // an extra quad, and its workgroup appends it to the cache.
    const int g = b % HKV, sp = b / HKV;
    const int nslot = kWaves * SP, ws = __builtin_amdgcn_readfirstlane(sp * kWaves + wave);
    const int nquad = (pos + 3) / 4, qbase = nquad / nslot, qextra = nquad % nslot;
    const int qa = ws * qbase + min(ws, qextra), qe = qa + qbase + (ws < qextra ? 1 : 0);
    const int ws_new = nslot - 1;
    const size_t kv_head_off = (size_t)g * a.max_ctx * kHeadDim;

    auto lblock = [&](int l) { return a.layer0 + (size_t)l * a.layer_stride; };
    // tags of this launch: ep + 1 .. ep + 8L + 6 (the zeroed words of a fresh arena never match)
    auto tag = [&](int l, int ph) { return ep + 8u * (uint32_t)l + (uint32_t)ph + 1u; };

    // ---- register prefetch state.  Each phase waits for its inputs, computes, publishes, and only then
    // issues the loads of a later phase: a burst of loads from every workgroup at once blocks the issuing wave
    // until the memory queues drain, so it belongs in the wait for the next inputs, not before a computation
    // that others are waiting for (and a poll, waiting for the vector memory counter, also waits for every
    // older load).
    // With eight KV heads (the attention of KV head g runs on workgroups b = g mod 8, which the dispatcher
    // places on XCD g), the Q/K/V rows of KV head g and the split merge of its query heads go to the same
    // workgroups' XCD: measured slightly faster.  Placement only: every exchange stays device-coherent.
    const bool xcd_local = HKV == 8 && G == 2;
    const int xrep = b & (kXwReps - 1);  // the copy of the all-gathered words this workgroup polls (its XCD's)
    int rq[RQ_MAX];
    bool rqv[RQ_MAX];
#pragma unroll
    for (int j = 0; j < RQ_MAX; ++j) {
        if (xcd_local) {  // the (G + 2) * 128 = 512 rows of KV head b mod 8 over the 128 waves of its XCD
            const int gx = b & 7, lr = (b >> 3) * kWaves + wave + (kNW / 8) * j;
            rq[j] = lr < G * kHeadDim ? gx * G * kHeadDim + lr
                                      : (lr < (G + 1) * kHeadDim ? q_dim + gx * kHeadDim + (lr - G * kHeadDim)
                                                                 : q_dim + kv_dim + gx * kHeadDim + (lr - (G + 1) * kHeadDim));
        } else {
            rq[j] = gw + kNW * j;
        }
        rqv[j] = rq[j] < Nqkv;
    }
    int ru[2 * RU_MAX];
    bool ruv[2 * RU_MAX];
#pragma unroll
    for (int j = 0; j < RU_MAX; ++j) {
        const int u = gw + kNW * j;
        ru[2 * j] = u;
        ru[2 * j + 1] = I + u;
        ruv[2 * j] = ruv[2 * j + 1] = u < I;
    }
    const int ro[1] = {gw};
    const bool rov[1] = {true};

    uint4 wq[RQ_MAX][CH];
    float sq[RQ_MAX][CH];
    uint4 wo[1][KO_MAX];
    float so[1][KO_MAX];
    uint4 wu[2 * RU_MAX][CH];
    float su[2 * RU_MAX][CH];
    uint4 wd[1][KD_MAX];
    float sd[1][KD_MAX];
    constexpr int CQ = chunk_quads<G>();
    uint4 kA[CQ], vA[CQ], kB[CQ], vB[CQ];  // cached K/V of the wave's first two chunks
    float nq[CH][E], nu[CH][E];  // RMSNorm weight slices of the Q and U phases
    float4 nq4, nu4;             // q8 x q8: the same weights for elements 4 tid .. 4 tid + 3 (quant_wg)
    float qkn[4], rcs[2];        // QK-Norm weights (q: lane, lane + 64; k: same) and this position's cos/sin

    // ---- prologue: layer-0 Q/K/V weights in flight, then the input vector (every workgroup builds it all)
    load_rows<Q8, RQ_MAX, CH>(a.layer0 + a.wqkv, (const float *)(a.layer0 + a.sqkv), kHid, rq, rqv, CH, lane, wq, sq);
    if constexpr (Q8 == 2)
        nq4 = *((const float4 *)(a.layer0 + a.attn_norm) + tid);
    else
        load_slice<Q8, CH>((const float *)(a.layer0 + a.attn_norm), lane, nq);
    if (a.token) {
        int tok = a.token[0];
        if (tok < 0 || tok >= a.V) {
            if (b == 0 && tid == 0) atomicOr(a.status, kStatusBadToken);
            tok = 0;
        }
        for (int k = tid; k < kHid; k += 256) {
            const size_t i = (size_t)tok * kHid + k;
            xs[padx(k)] = Q8 ? (float)((const int8_t *)a.embed)[i] * a.embed_scales[i >> 5]
                       : bf16_to_f32(((const uint16_t *)a.embed)[i]);
        }
    } else {
        for (int k = tid; k < kHid; k += 256) xs[padx(k)] = a.hidden_in[k];
    }
    __syncthreads();
    float x_own = xs[padx(gw)];  // residual stream of the owned row

    const int dsub = (lane & 15) * 8;
    // score scale 1/sqrt(128) applied to the finished dot product, in log2 units: exp(s - m) = 2^(s' - m')
    // with s' = s * log2(e)
    const float sl2 = (1.0f / sqrtf((float)kHeadDim)) * 1.4426950408889634f;

    for (int l = 0; l < a.L; ++l) {
        const uint8_t *lb = lblock(l);
        const uint16_t *kb = a.kcache + (size_t)l * a.kv_layer_stride + kv_head_off;
        const uint16_t *vb = a.vcache + (size_t)l * a.kv_layer_stride + kv_head_off;
        // ================= Q: RMSNorm + Q/K/V rows
        if (l > 0) {
            const uint64_t *src = a.xd + xrep * xw_rep(kHid);
            const bool ok = poll<4, true>([&](int i) { return src + xw_index(i); }, kHid, tag(l - 1, 5), xs, a.status);
            if (!all_ok(ok, s_fail, a.status)) return;
        }
        QW3_STAMP(l, 0, 0);
        {
            float d[RQ_MAX];
            if constexpr (Q8 == 2) {
                quant_wg<true>(xs, kHid, nq4, rms_inv(xs, a.eps, lane), qcode, qdsc);
                __syncthreads();
#pragma unroll
                for (int j = 0; j < RQ_MAX; ++j) d[j] = wave_sum_fast(dot_codes<CH>(wq[j], sq[j], qcode, qdsc, CH, lane));
            } else {
                float xr[CH][E];
                rms_slice<Q8, CH>(xs, nq, a.eps, lane, xr);
#pragma unroll
                for (int j = 0; j < RQ_MAX; ++j) d[j] = wave_sum_fast(dot_reg<Q8, CH>(wq[j], sq[j], xr));
            }
#pragma unroll
            for (int j = 0; j < RQ_MAX; ++j)
                if (lane == j && rqv[j]) put(a.qkv + rq[j], d[j], tag(l, 0));
        }
        QW3_STAMP(l, 0, 1);
        {  // attention-phase loads: QK-Norm weights, this position's RoPE row, the first cached group
            const float *qnw = (const float *)(lb + a.q_norm), *knw = (const float *)(lb + a.k_norm);
            qkn[0] = qnw[lane];
            qkn[1] = qnw[lane + 64];
            qkn[2] = knw[lane];
            qkn[3] = knw[lane + 64];
            rcs[0] = a.rope_cos[(size_t)pos * (kHeadDim / 2) + lane];
            rcs[1] = a.rope_sin[(size_t)pos * (kHeadDim / 2) + lane];
            load_chunk(kb, vb, qa, qe, pos, lane, kA, vA);
            // a second chunk (contexts past one chunk per wave slot) is in flight before the poll too, so no
            // wave waits for a load after its inputs arrive
            if (qa + CQ < qe) load_chunk(kb, vb, qa + CQ, qe, pos, lane, kB, vB);
        }

        // ================= A: QK-Norm + RoPE + append + attention over this split
        {
            float *raw = big;                                // [(G + 2) * 128]: q heads, k, v
            float *qs = big + 1024 + wave * G * kHeadDim;    // this wave's [G][128] normalised, rotated queries
            float *kn = big + 3072;                          // new key (bf16 value)
            float *vn = big + 3200;                          // new value (bf16 value)
            const uint64_t *qkv = a.qkv;
            const int hq0 = g * G;
            auto src = [&](int i) {
                const int h = i >> 7, d = i & 127;
                const int row = h < G ? (hq0 + h) * kHeadDim + d
                                      : (h == G ? q_dim + g * kHeadDim + d : q_dim + kv_dim + g * kHeadDim + d);
                return qkv + row;
            };
            const bool ok = poll<3>(src, (G + 2) * kHeadDim, tag(l, 0), raw, a.status);
            if (!all_ok(ok, s_fail, a.status)) return;
            QW3_STAMP(l, 1, 0);

            // QK-Norm ([P1] item 3, one 128-weight vector per projection) then RoPE on pairs (i, i + 64) at
            // `pos` (item 4), 1/sqrt on v_rsq_f32.  Every wave normalises the G query heads into LDS rows of its
            // own (read back by the same wave: no workgroup barrier); the key head and the value matter only to
            // the wave of the new position, which also appends both to the cache ([P1] section 6, rounded to the
            // cache's bf16).
            const float c = rcs[0], s = rcs[1];
            auto norm_rope = [&](int h, float w0, float w1, float &r0, float &r1) {
                const float v0 = raw[h * kHeadDim + lane], v1 = raw[h * kHeadDim + lane + 64];
                const float inv = __builtin_amdgcn_rsqf(wave_sum_fast(v0 * v0 + v1 * v1) / (float)kHeadDim + a.eps);
                const float n0 = w0 * (v0 * inv), n1 = w1 * (v1 * inv);
                r0 = n0 * c - n1 * s;
                r1 = n1 * c + n0 * s;
            };
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float r0, r1;
                norm_rope(h, qkn[0], qkn[1], r0, r1);
                qs[h * kHeadDim + lane] = r0;
                qs[h * kHeadDim + lane + 64] = r1;
            }
            if (ws == ws_new) {
                float r0, r1;
                norm_rope(G, qkn[2], qkn[3], r0, r1);
                const uint16_t k0 = f32_to_bf16(r0), k1 = f32_to_bf16(r1);
                const uint16_t v0b = f32_to_bf16(raw[(G + 1) * kHeadDim + lane]);
                const uint16_t v1b = f32_to_bf16(raw[(G + 1) * kHeadDim + lane + 64]);
                kn[lane] = bf16_to_f32(k0);
                kn[lane + 64] = bf16_to_f32(k1);
                vn[lane] = bf16_to_f32(v0b);
                vn[lane + 64] = bf16_to_f32(v1b);
                uint16_t *kc = (uint16_t *)kb + (size_t)pos * kHeadDim;
                uint16_t *vc = (uint16_t *)vb + (size_t)pos * kHeadDim;
                kc[lane] = k0;
                kc[lane + 64] = k1;
                vc[lane] = v0b;
                vc[lane + 64] = v1b;
            }

            float qr[G][8];
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int e = 0; e < 8; ++e) qr[h][e] = qs[h * kHeadDim + dsub + e];
            float m[G], lsum[G], acc[G][8];
#pragma unroll
            for (int h = 0; h < G; ++h) {
                m[h] = -INFINITY;
                lsum[h] = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
            }
            // the first two chunks were prefetched; later chunks (contexts past two chunks per wave slot)
            // stream one ahead
            attend_run<G>(kA, vA, qa, qe - qa, pos, lane, qr, sl2, m, lsum, acc);
            for (int q0 = qa + CQ; q0 < qe; q0 += CQ) {
                const bool more = q0 + CQ < qe;
                uint4 kN[CQ], vN[CQ];
                if (more) load_chunk(kb, vb, q0 + CQ, qe, pos, lane, kN, vN);
                attend_run<G>(kB, vB, q0, qe - q0, pos, lane, qr, sl2, m, lsum, acc);
                if (!more) break;
#pragma unroll
                for (int i = 0; i < CQ; ++i) {
                    kB[i] = kN[i];
                    vB[i] = vN[i];
                }
            }
            if (ws == ws_new) attend_new<G>(kn, vn, lane, qr, sl2, m, lsum, acc);
            // the four lane rows of each wave share the running max (wave-uniform), so their (l, acc) add up
            // directly: two register swaps across rows (lanes l, l + 32, then odd and even rows) fold the 8 G
            // values of a lane into 2 G, row r holding values r * 2G .. r * 2G + 2G - 1 of the flattened
            // [G][8] (one head, contiguous dims); one LDS pass then combines the four waves per output dim
            {
                constexpr int NV = 8 * G;
                float fv[NV];
#pragma unroll
                for (int h = 0; h < G; ++h)
#pragma unroll
                    for (int e = 0; e < 8; ++e) fv[h * 8 + e] = acc[h][e];
                float r1[NV / 2];
#pragma unroll
                for (int k = 0; k < NV / 2; ++k) {
                    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(fv[k]), __float_as_uint(fv[k + NV / 2]),
                                                                    false, false);
                    r1[k] = __uint_as_float(p[0]) + __uint_as_float(p[1]);
                }
                float r2[NV / 4];
#pragma unroll
                for (int k = 0; k < NV / 4; ++k) {
                    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(r1[k]), __float_as_uint(r1[k + NV / 4]),
                                                                    false, false);
                    r2[k] = __uint_as_float(p[0]) + __uint_as_float(p[1]);
                }
                const int r = lane >> 4, k0 = r * (NV / 4);
                float *wp = wacc + (wave * G + (k0 >> 3)) * kHeadDim + dsub + (k0 & 7);
                if constexpr (G == 1) {
                    *(float2 *)wp = make_float2(r2[0], r2[1]);
                } else {
#pragma unroll
                    for (int q = 0; q < NV / 16; ++q)
                        *(float4 *)(wp + 4 * q) = make_float4(r2[4 * q], r2[4 * q + 1], r2[4 * q + 2], r2[4 * q + 3]);
                }
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(lsum[h]), __float_as_uint(lsum[h]),
                                                                    false, false);
                    const float t = __uint_as_float(p[0]) + __uint_as_float(p[1]);
                    const auto p2 = __builtin_amdgcn_permlane16_swap(__float_as_uint(t), __float_as_uint(t), false, false);
                    const float lw = __uint_as_float(p2[0]) + __uint_as_float(p2[1]);
                    if (lane == 0) {
                        wl[wave][h] = lw;
                        wm[wave][h] = m[h];
                    }
                }
            }
            __syncthreads();
            uint64_t *pp = a.part + ((size_t)(g * SP + sp) * G) * PW;
            for (int t = tid; t < G * kHeadDim; t += 256) {
                const int h = t >> 7, d = t & 127;
                float M = -INFINITY;
#pragma unroll
                for (int w = 0; w < kWaves; ++w) M = fmaxf(M, wm[w][h]);
                float Ls = 0.f, O = 0.f;
                if (M != -INFINITY) {
#pragma unroll
                    for (int w = 0; w < kWaves; ++w) {
                        const float f = exp2_hw(wm[w][h] - M);
                        Ls += f * wl[w][h];
                        O += f * wacc[(w * G + h) * kHeadDim + d];
                    }
                }
                uint64_t *ph = pp + (size_t)h * PW;
                if (d == 0) {
                    put(ph, M, tag(l, 1));
                    put(ph + 1, Ls, tag(l, 1));
                }
                put(ph + 2 + d, O, tag(l, 1));
            }
        }
        QW3_STAMP(l, 1, 1);
        load_rows<Q8, 1, KO_MAX>(lb + a.wo, (const float *)(lb + a.so), q_dim, ro, rov, KO, lane, wo, so);

        // ================= M: merge of the context splits of one query head, dpw output dims per workgroup
        {
            const int wph = kMegaGrid / HQ;  // workgroups per query head
            const int dpw = kHeadDim / wph;  // dims per workgroup
            const int h = xcd_local ? (b & 7) * G + (b >> 3) / wph : b / wph;
            const int dc = xcd_local ? (b >> 3) % wph : b % wph;
            const int gh = h / G, hh = h % G;
            const int per = 2 + dpw;
            const uint64_t *part = a.part;
            auto src = [&](int i) {
                const int s = i / per, j = i % per;
                const size_t base = ((size_t)(gh * SP + s) * G + hh) * PW;
                return part + base + (j < 2 ? j : 2 + dc * dpw + (j - 2));
            };
            // SP * per = 512 / HKV + 128 G words at most (one KV head): (512 + 128 G) / 256 per thread
            static_assert(512 + 128 * G <= kMegaBuf, "merge inputs fit the LDS buffer");
            const bool ok = poll<(512 + 128 * G + 255) / 256>(src, SP * per, tag(l, 1), big, a.status);
            if (!all_ok(ok, s_fail, a.status)) return;
            QW3_STAMP(l, 2, 0);
            // exact combination (split order fixed by the reduction tree): M = max m_s,
            // o = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s, scores in log2 units
            if (SP <= 32 && dpw == 2 * kWaves) {
                // one pass: each half wave takes one dim, lane s of the half takes split s
                const int e = 2 * wave + (lane >> 5), s = lane & 31;
                const bool v = s < SP;
                const float ms = v ? big[s * per] : -INFINITY;
                const float ls = v ? big[s * per + 1] : 0.f, os = v ? big[s * per + 2 + e] : 0.f;
                const bool hi = lane >= 32;
                float r = row16_max(ms);
                const float M = hi ? fmaxf(lane_get(r, 32), lane_get(r, 48)) : fmaxf(lane_get(r, 0), lane_get(r, 16));
                const float f = ms == -INFINITY ? 0.f : exp2_hw(ms - M);
                const float rl = row16_sum(f * ls), ro = row16_sum(f * os);
                const float Ls = hi ? lane_get(rl, 32) + lane_get(rl, 48) : lane_get(rl, 0) + lane_get(rl, 16);
                const float O = hi ? lane_get(ro, 32) + lane_get(ro, 48) : lane_get(ro, 0) + lane_get(ro, 16);
                if ((lane & 31) < kXwReps)
                    put(a.attn + (lane & 31) * xw_rep(q_dim) + xw_index(h * kHeadDim + dc * dpw + e), O / Ls, tag(l, 2));
            } else {
                for (int e = wave; e < dpw; e += kWaves) {
                    float M = -INFINITY;
                    for (int s = lane; s < SP; s += 64) M = fmaxf(M, big[s * per]);
                    M = wave_max_fast(M);
                    float Ls = 0.f, O = 0.f;
                    for (int s = lane; s < SP; s += 64) {
                        const float ms = big[s * per];
                        const float f = ms == -INFINITY ? 0.f : exp2_hw(ms - M);
                        Ls += f * big[s * per + 1];
                        O += f * big[s * per + 2 + e];
                    }
                    Ls = wave_sum_fast(Ls);
                    O = wave_sum_fast(O);
                    if (lane < kXwReps)
                        put(a.attn + lane * xw_rep(q_dim) + xw_index(h * kHeadDim + dc * dpw + e), O / Ls, tag(l, 2));
                }
            }
        }
        QW3_STAMP(l, 2, 1);
        load_rows<Q8, 2 * RU_MAX, CH>(lb + a.wgu, (const float *)(lb + a.sgu), kHid, ru, ruv, CH, lane, wu, su);
        if constexpr (Q8 == 2)
            nu4 = *((const float4 *)(lb + a.mlp_norm) + tid);
        else
            load_slice<Q8, CH>((const float *)(lb + a.mlp_norm), lane, nu);
        // the down-projection rows go out here too, so the gate/up poll has no loads in front of it (its
        // inputs are the o_proj outputs, the layer's most contended exchange): 0.37 us per layer faster than
        // issuing them after o_proj.  Moving any other phase's weights one poll earlier measured slower.
        load_rows<Q8, 1, KD_MAX>(lb + a.wd, (const float *)(lb + a.sd), I, ro, rov, KD, lane, wd, sd);

        // ================= O: o_proj + residual on the owned row
        {
            const uint64_t *src = a.attn + xrep * xw_rep(q_dim);
            const bool ok = poll<8, true>([&](int i) { return src + xw_index(i); }, q_dim, tag(l, 2), big, a.status);
            if (!all_ok(ok, s_fail, a.status)) return;
            QW3_STAMP(l, 3, 0);
            if constexpr (Q8 == 2) {
                quant_wg<false>(big, q_dim, float4{}, 0.f, qcode, qdsc);
                __syncthreads();
            }
            const float d = wave_sum_fast(Q8 == 2 ? dot_codes<KO_MAX>(wo[0], so[0], qcode, qdsc, KO, lane)
                                                  : dot_lds<Q8, KO_MAX>(wo[0], so[0], big, KO, lane));
            x_own = x_own + d;
            if (lane < kXwReps) put(a.xo + lane * xw_rep(kHid) + xw_index(gw), x_own, tag(l, 3));
        }
        QW3_STAMP(l, 3, 1);

        // ================= U: RMSNorm + gate/up + SwiGLU
        {
            const uint64_t *src = a.xo + xrep * xw_rep(kHid);
            const bool ok = poll<4, true>([&](int i) { return src + xw_index(i); }, kHid, tag(l, 3), xs, a.status);
            if (!all_ok(ok, s_fail, a.status)) return;
            QW3_STAMP(l, 4, 0);
            float xr[CH][E];
            if constexpr (Q8 == 2) {
                quant_wg<true>(xs, kHid, nu4, rms_inv(xs, a.eps, lane), qcode, qdsc);
                __syncthreads();
            } else {
                rms_slice<Q8, CH>(xs, nu, a.eps, lane, xr);
            }
            float av[RU_MAX];
            auto udot = [&](int r) {
                if constexpr (Q8 == 2) {
                    return dot_codes<CH>(wu[r], su[r], qcode, qdsc, CH, lane);
                } else {
                    return dot_reg<Q8, CH>(wu[r], su[r], xr);
                }
            };
#pragma unroll
            for (int j = 0; j < RU_MAX; ++j) {
                const float gt = wave_sum_fast(udot(2 * j));
                const float up = wave_sum_fast(udot(2 * j + 1));
                // SwiGLU, [P1] section 5: (g * sigmoid(g)) * u with sigmoid(g) = 1 / (1 + exp(-g)), on the
                // transcendental unit (2^x and reciprocal, each within about 1 ulp)
                const float sig = __builtin_amdgcn_rcpf(1.0f + exp2_hw(-gt * 1.4426950408889634f));
                av[j] = (gt * sig) * up;
            }
#pragma unroll
            for (int j = 0; j < RU_MAX; ++j)
                if (lane < kXwReps && ruv[2 * j]) put(a.act + lane * xw_rep(I) + xw_index(ru[2 * j]), av[j], tag(l, 4));
        }
        QW3_STAMP(l, 4, 1);
        if (l + 1 < a.L) {
            const uint8_t *nb = lblock(l + 1);
            load_rows<Q8, RQ_MAX, CH>(nb + a.wqkv, (const float *)(nb + a.sqkv), kHid, rq, rqv, CH, lane, wq, sq);
            if constexpr (Q8 == 2)
                nq4 = *((const float4 *)(nb + a.attn_norm) + tid);
            else
                load_slice<Q8, CH>((const float *)(nb + a.attn_norm), lane, nq);
        }

        // ================= D: down + residual on the owned row
        {
            const uint64_t *src = a.act + xrep * xw_rep(I);
            const bool ok = poll<kMegaBuf / 256, true>([&](int i) { return src + xw_index(i); }, I, tag(l, 4), big, a.status);
            if (!all_ok(ok, s_fail, a.status)) return;
            QW3_STAMP(l, 5, 0);
            if constexpr (Q8 == 2) {
                quant_wg<false>(big, I, float4{}, 0.f, qcode, qdsc);
                __syncthreads();
            }
            const float d = wave_sum_fast(Q8 == 2 ? dot_codes<KD_MAX>(wd[0], sd[0], qcode, qdsc, KD, lane)
                                                  : dot_lds<Q8, KD_MAX>(wd[0], sd[0], big, KD, lane));
            x_own = x_own + d;
            if (l + 1 < a.L) {
                if (lane < kXwReps) put(a.xd + lane * xw_rep(kHid) + xw_index(gw), x_own, tag(l, 5));
            } else if (lane == 0) {
                a.x_out[gw] = x_own;
            }
        }
        QW3_STAMP(l, 5, 1);
    }
    // Every workgroup read the epoch before its first phase, and workgroup 0 has consumed every workgroup's
    // output since, so the next launch's tag base can be published now.
    if (b == 0 && tid == 0) a.epoch[0] = ep + (uint32_t)(8 * a.L + 8);
}

#ifdef QW3_MEGA_STAMPS
// Copies the phase-stamp table of the last launch (layers x 6 phases x 2 x kMegaGrid uint64, 100 MHz ticks).
extern "C" int32_t qw3_mega_stamps(void *host_out, uint64_t bytes) {
    if (!host_out || bytes < sizeof(uint64_t) * (uint64_t)kStampLayers * 6 * 2 * kMegaGrid) return QW3_INVALID_ARGUMENT;
    return hipMemcpyFromSymbol(host_out, HIP_SYMBOL(g_mega_stamps), sizeof(uint64_t) * (size_t)kStampLayers * 6 * 2 *
                               kMegaGrid) == hipSuccess ? QW3_OK : QW3_DEVICE_ERROR;
}
#endif

bool mega_supported(const Dims &d) {
    if (d.H != kHid || d.S < 1) return false;
    if (d.HKV < 2 || kMegaGrid % d.HKV || d.HQ > 16 || kMegaGrid % d.HQ) return false;
    // merge phase inputs: every split partial of a KV head, (2 + dims per workgroup) words each
    const int npart = kMegaGrid / d.HKV, dpw = kHeadDim / (kMegaGrid / d.HQ);
    if (npart * (2 + dpw) > kMegaBuf) return false;
    if (d.q_dim + 2 * d.HKV * kHeadDim > 4 * kNW) return false;
    if (d.I > 3 * kNW || d.I % (d.q8 ? 1024 : 512)) return false;
    if (d.q_dim % (d.q8 ? 1024 : 512)) return false;
    return true;
}

// The persistent grid must be resident all at once: every workgroup waits for the others' outputs.  True when
// the current device holds at least kMegaGrid of these workgroups at one time (compute units times the
// occupancy the kernel's registers and LDS allow).  A device that cannot (fewer compute units, a partitioned
// GPU) takes the kernel-by-kernel path instead.
bool mega_resident(int wmode, int G) {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return false;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return false;
    const void *fn = nullptr;
#define QW3_MEGA_FN(Q, GG) fn = reinterpret_cast<const void *>(&decode_mega_kernel<Q, GG>)
    if (wmode == 2) {
        if (G == 1) QW3_MEGA_FN(2, 1);
        else if (G == 2) QW3_MEGA_FN(2, 2);
        else if (G == 4) QW3_MEGA_FN(2, 4);
    } else if (wmode == 1) {
        if (G == 1) QW3_MEGA_FN(1, 1);
        else if (G == 2) QW3_MEGA_FN(1, 2);
        else if (G == 4) QW3_MEGA_FN(1, 4);
    } else {
        if (G == 1) QW3_MEGA_FN(0, 1);
        else if (G == 2) QW3_MEGA_FN(0, 2);
        else if (G == 4) QW3_MEGA_FN(0, 4);
    }
#undef QW3_MEGA_FN
    if (!fn) return false;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kMegaWaves * 64, 0) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    return (long long)per_cu * cus >= kMegaGrid;
}

hipError_t launch_decode_mega(int wmode, int G, const MegaArgs &a, hipStream_t st) {
    const dim3 grid(kMegaGrid), block(kWaves * 64);
#define QW3_MEGA(Q, GG) hipLaunchKernelGGL((decode_mega_kernel<Q, GG>), grid, block, 0, st, a)
    if (wmode == 2) {
        switch (G) {
            case 1: QW3_MEGA(2, 1); break;
            case 2: QW3_MEGA(2, 2); break;
            case 4: QW3_MEGA(2, 4); break;
            default: return hipErrorInvalidValue;
        }
    } else if (wmode == 1) {
        switch (G) {
            case 1: QW3_MEGA(1, 1); break;
            case 2: QW3_MEGA(1, 2); break;
            case 4: QW3_MEGA(1, 4); break;
            default: return hipErrorInvalidValue;
        }
    } else {
        switch (G) {
            case 1: QW3_MEGA(0, 1); break;
            case 2: QW3_MEGA(0, 2); break;
            case 4: QW3_MEGA(0, 4); break;
            default: return hipErrorInvalidValue;
        }
    }
#undef QW3_MEGA
    return hipGetLastError();
}

}  // namespace qw3
