// Deterministic token sampling on gfx950 over up to 16 rows of logits.
//
// The sampling order of [P4] "Sampling order" (with [P1] section 7):
//   forbidden tokens -> -inf; repetition penalty on tokens present in the history (positive logits divided by
//   the penalty, negative ones multiplied; each token once); NaN -> -inf; -0 -> +0; a +inf logit is a
//   numerical failure; temperature 0 -> the greatest logit, lowest id on ties, no draw; otherwise divide by
//   the temperature, keep the top-k by (value desc, id asc), stable probabilities over them, order by
//   (probability desc, id asc), keep the shortest prefix whose cumulative probability reaches top-p,
//   re-normalise it and draw with PCG32 ([P4] "Deterministic sampling contract"): the first candidate whose
//   cumulative probability exceeds u = (word >> 8) * 2^-24.
//
// Two launches, no atomics across workgroups and no memset (every scratch word a launch reads was written by
// the previous launch of the same call):
//   sample_chunk_kernel   grid (kSampleChunks, rows): one workgroup per slice of the vocabulary applies the
//                         transforms in registers, keeps the slice's keys in LDS and selects its exact top-k
//                         (radix select, 8 bits per pass, ties at the threshold taken in id order), writing them
//                         in id order to scratch;
//   sample_finish_kernel  grid (rows): merges the slices' candidates the same way, sorts the k survivors in LDS
//                         (bitonic), and runs the probability, top-p and draw steps.  Every floating-point sum of
//                         those steps is taken by one thread in the candidates' order, exactly as the steps state
//                         them, so the result does not depend on the launch shape.
//
// Page titles used in citations:
//   [P1] "Scalar-Native Qwen3 Reference Runtime As The Numerical Authority"
//   [P4] "Portable WebAssembly Runtime Architecture for TinyRustLM"
#include <math.h>

#include <mutex>

#include "common.h"

namespace qw3 {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kChunkMax = kSampleMaxVocab / kSampleChunks;  // vocabulary slice per chunk workgroup
constexpr int kMergeMax = kSampleChunks * kSampleMaxTopK;   // candidates the finishing workgroup merges

// Float -> unsigned key with the same order (finite values); 0 is reserved for -inf (never a candidate).
__device__ __forceinline__ uint32_t f2key(float f) {
    if (f == -INFINITY) return 0u;
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key2f(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__device__ __forceinline__ int wave_incl_scan(int v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(v, o, 64);
        if (lane >= o) v += t;
    }
    return v;
}

// Exclusive prefix sum of one int per thread over the workgroup (thread order); *total gets the sum.
// s_w: kWaves + 1 ints of LDS.  Ends with a barrier, so s_w may be reused right after.
__device__ int block_excl_scan(int v, int *s_w, int *total) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int inc = wave_incl_scan(v);
    if (lane == 63) s_w[w] = inc;
    __syncthreads();
    if (tid < 64) {
        const int x = tid < kWaves ? s_w[tid] : 0;
        const int xi = wave_incl_scan(x);
        if (tid < kWaves) s_w[tid] = xi - x;
        if (tid == kWaves - 1) s_w[kWaves] = xi;
    }
    __syncthreads();
    const int r = s_w[w] + inc - v;
    *total = s_w[kWaves];
    __syncthreads();
    return r;
}

// The k-th largest nonzero key among key_at(0..n) (1 <= k <= number of nonzero keys): returns the threshold
// key T and how many elements equal to T belong to the top k (the others are strictly greater).  Four
// passes of 8 bits; per pass one LDS histogram, and wave 0 finds the bin where the count from the top
// reaches k.
template <typename KeyAt>
__device__ void radix_select(KeyAt key_at, int n, int k, uint32_t *hist, int *s_res, uint32_t &T, int &need) {
    const int tid = threadIdx.x, lane = tid & 63;
    uint32_t prefix = 0, mask = 0;
    int rem = k;
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        if (tid < 256) hist[tid] = 0;
        __syncthreads();
        for (int i = tid; i < n; i += kThreads) {
            const uint32_t key = key_at(i);
            if (key && (key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (tid < 64) {
            // lane l holds bins 255-4l .. 252-4l, i.e. the bins in descending order, four per lane
            uint32_t c[4], S = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                c[j] = hist[255 - 4 * lane - j];
                S += c[j];
            }
            const int inc = wave_incl_scan((int)S);
            const uint32_t P = (uint32_t)inc - S;
            if (P < (uint32_t)rem && (uint32_t)rem <= P + S) {
                uint32_t acc = P;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (acc + c[j] >= (uint32_t)rem) {
                        s_res[0] = 255 - 4 * lane - j;
                        s_res[1] = rem - (int)acc;
                        break;
                    }
                    acc += c[j];
                }
            }
        }
        __syncthreads();
        prefix |= (uint32_t)s_res[0] << shift;
        mask |= 0xffu << shift;
        rem = s_res[1];
        __syncthreads();
    }
    T = prefix;
    need = rem;
}

// Sorts a[0..P) (P a power of two <= kThreads) in descending order.
__device__ void bitonic_desc(uint64_t *a, int P) {
    const int i = threadIdx.x;
    for (int size = 2; size <= P; size <<= 1)
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            if (i < P) {
                const int j = i ^ stride;
                if (j > i) {
                    const uint64_t x = a[i], y = a[j];
                    const bool desc = (i & size) == 0;
                    if (desc ? x < y : x > y) {
                        a[i] = y;
                        a[j] = x;
                    }
                }
            }
            __syncthreads();
        }
}

__host__ __device__ __forceinline__ uint32_t pcg32_next(uint64_t &state, uint64_t inc) {
    const uint64_t old = state;
    state = old * 6364136223846793005ull + inc;
    const uint32_t xs = (uint32_t)(((old >> 18) ^ old) >> 27), rot = (uint32_t)(old >> 59);
    return (xs >> rot) | (xs << ((32u - rot) & 31u));
}

__device__ __forceinline__ uint64_t shfl_xor64(uint64_t v, int m) {
    const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, m, 64), hi = (uint32_t)__shfl_xor((int)(v >> 32), m, 64);
    return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t readlane64(uint64_t v, int l) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(v >> 32), l);
    return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ float readlane_f(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// The 64 values of a wave (one per lane) sorted in descending order across the lanes: the bitonic network of
// bitonic_desc with each compare-exchange between lane i and lane i ^ stride done in registers.
__device__ __forceinline__ uint64_t wave_sort_desc(uint64_t v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int size = 2; size <= 64; size <<= 1)
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            const uint64_t o = shfl_xor64(v, stride);
            const bool keep_max = ((lane & size) == 0) == ((lane & stride) == 0);
            v = keep_max ? (v > o ? v : o) : (v < o ? v : o);
        }
    return v;
}

// The steps after the top-k selection for up to 64 survivors, in wave 0: lane j holds candidate v = (key << 32 |
// ~id) (0 past the survivors).  The same operations in the same order as the workgroup path below: every sum
// runs over the candidates one by one (readlane), so the drawn token is the same.
__device__ void finish_in_wave(const SampleArgs &a, int row, int k, uint64_t v) {
    const int lane = threadIdx.x & 63;
    v = wave_sort_desc(v);  // (value desc, id asc)
    auto set_outputs = [&](int tok) {
        if (lane == 0) {
            a.token_out[row] = tok;
            int done = 0;
            for (int j = 0; j < a.n_stop; ++j) done |= a.stop[j] == tok;
            if (a.done_out) a.done_out[row] = done;
            if (a.status_out) a.status_out[row] = QW3_OK;
        }
    };
    if (a.temperature == 0.f) {  // greedy: the greatest logit, lowest id on ties; no draw
        set_outputs((int)(0xffffffffu - (uint32_t)readlane64(v, 0)));
        return;
    }
    // stable probabilities over the k survivors ([P1] section 7)
    const float m = key2f((uint32_t)(readlane64(v, 0) >> 32));
    float e = 0.f;
    const uint32_t id = 0xffffffffu - (uint32_t)v;
    if (lane < k) e = (float)exp((double)(key2f((uint32_t)(v >> 32)) - m));
    float s = 0.f;
    for (int j = 0; j < k; ++j) s = s + readlane_f(e, j);
    uint64_t w = lane < k ? ((uint64_t)__float_as_uint(e / s) << 32) | (uint64_t)(0xffffffffu - id) : 0ull;
    w = wave_sort_desc(w);  // (probability desc, id asc)
    const float pw = __uint_as_float((uint32_t)(w >> 32));
    // top-p: the shortest prefix whose cumulative probability is at least p ([P4] "Sampling order")
    float cum = 0.f;
    int keep = k;
    for (int j = 0; j < k; ++j) {
        cum = cum + readlane_f(pw, j);
        if (cum >= a.top_p) {
            keep = j + 1;
            break;
        }
    }
    float s2 = 0.f;
    for (int j = 0; j < keep; ++j) s2 = s2 + readlane_f(pw, j);
    const float pr = lane < keep ? pw / s2 : 0.f;
    uint64_t st = a.rng[2 * row];
    const uint64_t inc = a.rng[2 * row + 1];
    const float u = (float)(pcg32_next(st, inc) >> 8) * (1.0f / 16777216.0f);
    float c2 = 0.f;
    int pick = keep - 1;
    for (int j = 0; j < keep; ++j) {
        c2 = c2 + readlane_f(pr, j);
        if (c2 > u) {
            pick = j;
            break;
        }
    }
    const uint64_t chosen = readlane64(w, pick);
    if (lane == 0) a.rng[2 * row] = st;
    set_outputs((int)(0xffffffffu - (uint32_t)chosen));
}

}  // namespace

__global__ __launch_bounds__(kThreads) void sample_chunk_kernel(SampleArgs a) {
    __shared__ uint32_t keys[kChunkMax];
    __shared__ uint32_t hbits[kChunkMax / 32], fbits[kChunkMax / 32];
    __shared__ uint32_t hist[256];
    __shared__ int s_w[kWaves + 1], s_res[2], s_bad;
    const int tid = threadIdx.x, row = blockIdx.y, c = blockIdx.x;
    const int chunk = (a.V + kSampleChunks - 1) / kSampleChunks;
    const int c0 = c * chunk, n = max(0, min(chunk, a.V - c0));
    for (int i = tid; i < kChunkMax / 32; i += kThreads) hbits[i] = fbits[i] = 0;
    if (tid == 0) s_bad = 0;
    __syncthreads();
    // tokens of this slice present in the row's history, and forbidden tokens
    for (int j = tid; j < a.n_history; j += kThreads) {
        const int t = a.history[(size_t)row * a.n_history + j] - c0;
        if (t >= 0 && t < n) atomicOr(&hbits[t >> 5], 1u << (t & 31));
    }
    for (int j = tid; j < a.n_forbid; j += kThreads) {
        const int t = a.forbid[j] - c0;
        if (t >= 0 && t < n) atomicOr(&fbits[t >> 5], 1u << (t & 31));
    }
    __syncthreads();
    // transforms, each thread on a contiguous run of the slice (so a scan in thread order is id order)
    const int run = (n + kThreads - 1) / kThreads;
    const int i0 = min(tid * run, n), i1 = min(i0 + run, n);
    const float *lg = a.logits + (size_t)row * a.ld + c0;
    int valid = 0;
    bool bad = false;
    for (int i = i0; i < i1; ++i) {
        float z = lg[i];
        if ((fbits[i >> 5] >> (i & 31)) & 1u) z = -INFINITY;
        if ((hbits[i >> 5] >> (i & 31)) & 1u) {
            if (z > 0.f) z = z / a.penalty;
            else if (z < 0.f) z = z * a.penalty;
        }
        if (z != z) z = -INFINITY;
        if (z == 0.f) z = 0.f;
        if (z == INFINITY) bad = true;
        if (a.temperature > 0.f) {
            z = z / a.temperature;
            if (z == INFINITY) bad = true;
        }
        const uint32_t key = f2key(z);
        keys[i] = key;
        valid += key != 0u;
    }
    if (bad) s_bad = 1;
    int n_valid;
    (void)block_excl_scan(valid, s_w, &n_valid);
    const int kc = min(a.top_k, n_valid);
    uint32_t *ck = a.cand_key + ((size_t)row * kSampleChunks + c) * kSampleMaxTopK;
    int *ci = a.cand_id + ((size_t)row * kSampleChunks + c) * kSampleMaxTopK;
    if (kc > 0) {
        uint32_t T;
        int need;
        radix_select([&](int i) { return keys[i]; }, n, kc, hist, s_res, T, need);
        int ties = 0;
        for (int i = i0; i < i1; ++i) ties += keys[i] == T;
        int dummy;
        int tr = block_excl_scan(ties, s_w, &dummy);
        int sel = 0;
        {
            int t2 = tr;
            for (int i = i0; i < i1; ++i) {
                const uint32_t k = keys[i];
                if (k > T) ++sel;
                else if (k == T && t2++ < need) ++sel;
            }
        }
        int pos = block_excl_scan(sel, s_w, &dummy);
        for (int i = i0; i < i1; ++i) {
            const uint32_t k = keys[i];
            bool s = k > T;
            if (k == T) s = tr++ < need;
            if (s && pos < kc) {  // exactly kc are selected; the bound only keeps a slip inside the block
                ck[pos] = k;
                ci[pos] = c0 + i;
                ++pos;
            }
        }
    }
    if (tid == 0) {
        a.cand_cnt[row * kSampleChunks + c] = kc;
        a.chunk_bad[row * kSampleChunks + c] = s_bad;
    }
}

__global__ __launch_bounds__(kThreads) void sample_finish_kernel(SampleArgs a) {
    __shared__ uint32_t keys[kMergeMax];
    __shared__ uint64_t srt[kSampleMaxTopK];
    __shared__ uint32_t hist[256];
    __shared__ int off[kSampleChunks + 1];
    __shared__ int s_w[kWaves + 1], s_res[2], s_keep;
    __shared__ float s_sum;
    const int tid = threadIdx.x, row = blockIdx.x;
    const uint32_t *ck = a.cand_key + (size_t)row * kSampleChunks * kSampleMaxTopK;
    const int *ci = a.cand_id + (size_t)row * kSampleChunks * kSampleMaxTopK;
    static_assert(kSampleChunks <= 64, "one wave gathers the slices' counts");
    if (tid < 64) {  // candidate counts of the slices -> offsets (a scan in slice order), and any failure
        const int cnt = tid < kSampleChunks ? a.cand_cnt[row * kSampleChunks + tid] : 0;
        const int bad = tid < kSampleChunks ? a.chunk_bad[row * kSampleChunks + tid] : 0;
        const int inc = wave_incl_scan(cnt);
        if (tid < kSampleChunks) off[tid] = inc - cnt;
        if (tid == kSampleChunks - 1) off[kSampleChunks] = inc;
        const uint64_t any_bad = __ballot(bad != 0);
        if (tid == 0) s_res[0] = any_bad != 0;
    }
    __syncthreads();
    const int n = off[kSampleChunks];
    if (s_res[0] || n == 0) {  // a +inf logit, or no finite one: numerical failure, nothing drawn
        if (tid == 0) {
            a.token_out[row] = -1;
            if (a.done_out) a.done_out[row] = 0;
            if (a.status_out) a.status_out[row] = QW3_NUMERICAL_FAILURE;
        }
        return;
    }
    // the slices' candidates, slice after slice: ascending token id
    for (int i = tid; i < n; i += kThreads) {
        int c = 0;  // the slice holding merged position i
#pragma unroll
        for (int j = 1; j < kSampleChunks; ++j) c += off[j] <= i;
        keys[i] = ck[(size_t)c * kSampleMaxTopK + (i - off[c])];
    }
    __syncthreads();
    const int k = min(a.top_k, n);
    uint32_t T;
    int need;
    radix_select([&](int i) { return keys[i]; }, n, k, hist, s_res, T, need);
    const int run = (n + kThreads - 1) / kThreads;
    const int i0 = min(tid * run, n), i1 = min(i0 + run, n);
    int ties = 0;
    for (int i = i0; i < i1; ++i) ties += keys[i] == T;
    int dummy;
    int tr = block_excl_scan(ties, s_w, &dummy);
    int sel = 0;
    {
        int t2 = tr;
        for (int i = i0; i < i1; ++i) {
            const uint32_t kk = keys[i];
            if (kk > T) ++sel;
            else if (kk == T && t2++ < need) ++sel;
        }
    }
    int pos = block_excl_scan(sel, s_w, &dummy);
    int P = 1;
    while (P < k) P <<= 1;
    for (int i = tid; i < P; i += kThreads) srt[i] = 0;
    __syncthreads();
    {
        int c = 0;
        while (c + 1 < kSampleChunks && off[c + 1] <= i0) ++c;
        for (int i = i0; i < i1; ++i) {
            while (off[c + 1] <= i) ++c;
            const uint32_t kk = keys[i];
            bool s = kk > T;
            if (kk == T) s = tr++ < need;
            if (s && pos < k) {  // exactly k are selected (see sample_chunk_kernel)
                const uint32_t id = (uint32_t)ci[(size_t)c * kSampleMaxTopK + (i - off[c])];
                srt[pos++] = ((uint64_t)kk << 32) | (uint64_t)(0xffffffffu - id);
            }
        }
    }
    __syncthreads();
    if (P <= 64) {  // up to 64 survivors: the rest runs in wave 0, one candidate per lane, no barriers
        if (tid < 64) finish_in_wave(a, row, k, tid < P ? srt[tid] : 0ull);
        return;
    }
    bitonic_desc(srt, P);  // (value desc, id asc)
    if (a.temperature == 0.f) {  // greedy: the greatest logit, lowest id on ties; no draw
        if (tid == 0) {
            const int tok = (int)(0xffffffffu - (uint32_t)srt[0]);
            a.token_out[row] = tok;
            int done = 0;
            for (int j = 0; j < a.n_stop; ++j) done |= a.stop[j] == tok;
            if (a.done_out) a.done_out[row] = done;
            if (a.status_out) a.status_out[row] = QW3_OK;
        }
        return;
    }
    // stable probabilities over the k survivors ([P1] section 7): subtract the maximum, exponentiate (in
    // double, one rounding to f32), sum in candidate order, divide
    float e = 0.f;
    uint32_t id = 0;
    if (tid < k) {
        const float m = key2f((uint32_t)(srt[0] >> 32));
        const float z = key2f((uint32_t)(srt[tid] >> 32));
        id = 0xffffffffu - (uint32_t)srt[tid];
        e = (float)exp((double)(z - m));
        keys[tid] = __float_as_uint(e);
    }
    __syncthreads();
    if (tid == 0) {
        float s = 0.f;
        for (int j = 0; j < k; ++j) s = s + __uint_as_float(keys[j]);
        s_sum = s;
    }
    __syncthreads();
    if (tid < P) srt[tid] = 0;
    __syncthreads();
    if (tid < k) srt[tid] = ((uint64_t)__float_as_uint(e / s_sum) << 32) | (uint64_t)(0xffffffffu - id);
    __syncthreads();
    bitonic_desc(srt, P);  // (probability desc, id asc)
    if (tid == 0) {
        // top-p: the shortest prefix whose cumulative probability is at least p ([P4] "Sampling order")
        float cum = 0.f;
        int keep = k;
        for (int j = 0; j < k; ++j) {
            cum = cum + __uint_as_float((uint32_t)(srt[j] >> 32));
            if (cum >= a.top_p) {
                keep = j + 1;
                break;
            }
        }
        float s2 = 0.f;
        for (int j = 0; j < keep; ++j) s2 = s2 + __uint_as_float((uint32_t)(srt[j] >> 32));
        s_keep = keep;
        s_sum = s2;
    }
    __syncthreads();
    const int keep = s_keep;
    if (tid < keep) keys[tid] = __float_as_uint(__uint_as_float((uint32_t)(srt[tid] >> 32)) / s_sum);
    __syncthreads();
    if (tid == 0) {
        uint64_t st = a.rng[2 * row];
        const uint64_t inc = a.rng[2 * row + 1];
        const float u = (float)(pcg32_next(st, inc) >> 8) * (1.0f / 16777216.0f);
        float cum = 0.f;
        int pick = keep - 1;
        for (int j = 0; j < keep; ++j) {
            cum = cum + __uint_as_float(keys[j]);
            if (cum > u) {
                pick = j;
                break;
            }
        }
        const int tok = (int)(0xffffffffu - (uint32_t)srt[pick]);
        a.rng[2 * row] = st;
        a.token_out[row] = tok;
        int done = 0;
        for (int j = 0; j < a.n_stop; ++j) done |= a.stop[j] == tok;
        if (a.done_out) a.done_out[row] = done;
        if (a.status_out) a.status_out[row] = QW3_OK;
    }
}

uint64_t sample_scratch_bytes(int rows) {
    const uint64_t per_row = (uint64_t)kSampleChunks * kSampleMaxTopK * 8 + (uint64_t)kSampleChunks * 8;
    return ((per_row * (uint64_t)rows) + 255) & ~uint64_t(255);
}

void sample_bind_scratch(SampleArgs &a, void *scratch) {
    uint8_t *p = (uint8_t *)scratch;
    const size_t n = (size_t)a.rows * kSampleChunks;
    a.cand_key = (uint32_t *)p;
    a.cand_id = (int *)(p + n * kSampleMaxTopK * 4);
    a.cand_cnt = (int *)(p + n * kSampleMaxTopK * 8);
    a.chunk_bad = a.cand_cnt + n;
}

hipError_t launch_sample(const SampleArgs &a, hipStream_t st) {
    hipLaunchKernelGGL(sample_chunk_kernel, dim3(kSampleChunks, a.rows), dim3(kThreads), 0, st, a);
    hipLaunchKernelGGL(sample_finish_kernel, dim3(a.rows), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace qw3

// ---- allocation-free variant ---------------------------------------------------------------------------
// For callers that cannot allocate (code under graph capture, tight serving loops, harnesses that forbid
// hipMalloc): qw3_sample_noalloc keeps the candidate scratch in this file-scope device array, one copy per GPU
// for as long as the process lives, sized for the largest request (QW3_SAMPLE_MAX_ROWS rows; the layout does
// not depend on the vocabulary).  Host code never passes the array's name to a kernel: the device address of
// each GPU's copy comes from hipGetSymbolAddress, taken once per device with that device current.
constexpr uint64_t kNoAllocScratchBytes =
    (((uint64_t)qw3::kSampleChunks * qw3::kSampleMaxTopK * 8 + (uint64_t)qw3::kSampleChunks * 8) *
         qw3::kSampleMaxRows +
     255) &
    ~uint64_t(255);
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of the current GPU's copy of `scratch` (looked up on the first call on that device).
int32_t noalloc_scratch(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return QW3_DEVICE_ERROR;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return QW3_DEVICE_ERROR;
        }
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return QW3_OK;
}
}  // namespace

// ---- C ABI ------------------------------------------------------------------------------------------------
namespace {

using namespace qw3;

// Host-side checks of qw3_sample's arguments; fills everything but the scratch pointers.
int32_t sample_args(SampleArgs &a, const float *logits, int32_t rows, int32_t V, int64_t ld,
                    const qw3_sample_params_t *p, const int32_t *history, int32_t n_history, const int32_t *forbid,
                    int32_t n_forbid, const int32_t *stop, int32_t n_stop, uint64_t *rng, int32_t *token_out,
                    int32_t *done_out, int32_t *status_out) {
    if (!logits || !p || !token_out || rows < 1 || rows > kSampleMaxRows || V < 1 || V > kSampleMaxVocab || ld < V)
        return QW3_INVALID_ARGUMENT;
    if (n_history < 0 || (n_history > 0 && !history) || n_forbid < 0 || (n_forbid > 0 && !forbid)) return QW3_INVALID_ARGUMENT;
    if (n_stop < 0 || n_stop > kSampleMaxStop || (n_stop > 0 && !stop)) return QW3_INVALID_ARGUMENT;
    if (!(p->repetition_penalty > 0.f) || isinf(p->repetition_penalty)) return QW3_INVALID_ARGUMENT;
    if (!(p->temperature >= 0.f) || isinf(p->temperature)) return QW3_INVALID_ARGUMENT;
    const bool draw = p->temperature > 0.f;
    if (draw && (p->top_k < 1 || p->top_k > kSampleMaxTopK || !(p->top_p > 0.f) || !(p->top_p <= 1.f) || !rng))
        return QW3_INVALID_ARGUMENT;
    a = SampleArgs{};
    a.logits = logits;
    a.ld = ld;
    a.V = V;
    a.rows = rows;
    a.temperature = p->temperature;
    a.top_p = p->top_p;
    a.penalty = p->repetition_penalty;
    a.top_k = draw ? p->top_k : 1;
    a.history = history;
    a.n_history = n_history;
    a.forbid = forbid;
    a.n_forbid = n_forbid;
    for (int i = 0; i < n_stop; ++i) a.stop[i] = stop[i];
    a.n_stop = n_stop;
    a.rng = rng;
    a.token_out = token_out;
    a.done_out = done_out;
    a.status_out = status_out;
    return QW3_OK;
}

}  // namespace

extern "C" {

int32_t qw3_pcg32_seed(uint64_t seed, uint64_t stream_id, uint64_t *state_out) {
    if (!state_out) return QW3_INVALID_ARGUMENT;
    uint64_t st = 0;
    const uint64_t inc = (stream_id << 1) | 1u;
    (void)pcg32_next(st, inc);
    st += seed;
    (void)pcg32_next(st, inc);
    state_out[0] = st;
    state_out[1] = inc;
    return QW3_OK;
}

int32_t qw3_sample_workspace_bytes(int32_t n_rows, uint64_t *bytes_out) {
    if (!bytes_out || n_rows < 1 || n_rows > kSampleMaxRows) return QW3_INVALID_ARGUMENT;
    *bytes_out = sample_scratch_bytes(n_rows);
    return QW3_OK;
}

int32_t qw3_sample(const float *logits_dev, int32_t n_rows, int32_t vocab, int64_t ld_logits,
                   const qw3_sample_params_t *params, const int32_t *history_dev, int32_t n_history,
                   const int32_t *forbid_dev, int32_t n_forbid, const int32_t *stop_ids, int32_t n_stop,
                   uint64_t *rng_dev, int32_t *token_out_dev, int32_t *done_out_dev, int32_t *status_out_dev,
                   void *workspace_dev, uint64_t workspace_bytes, void *stream) {
    SampleArgs a;
    const int32_t rc = sample_args(a, logits_dev, n_rows, vocab, ld_logits, params, history_dev, n_history, forbid_dev,
                                   n_forbid, stop_ids, n_stop, rng_dev, token_out_dev, done_out_dev, status_out_dev);
    if (rc != QW3_OK) return rc;
    if (!workspace_dev) return QW3_INVALID_ARGUMENT;
    if ((uintptr_t)workspace_dev & 255u) return QW3_ALIGNMENT;
    if (workspace_bytes < sample_scratch_bytes(n_rows)) return QW3_OUT_OF_MEMORY;
    sample_bind_scratch(a, workspace_dev);
    return launch_sample(a, (hipStream_t)stream) == hipSuccess ? QW3_OK : QW3_DEVICE_ERROR;
}

int32_t qw3_sample_noalloc(const float *logits_dev, int32_t n_rows, int32_t vocab, int64_t ld_logits,
                           const qw3_sample_params_t *params, const int32_t *history_dev, int32_t n_history,
                           const int32_t *forbid_dev, int32_t n_forbid, const int32_t *stop_ids, int32_t n_stop,
                           uint64_t *rng_dev, int32_t *token_out_dev, int32_t *done_out_dev, int32_t *status_out_dev,
                           void *stream) {
    SampleArgs a;
    const int32_t rc = sample_args(a, logits_dev, n_rows, vocab, ld_logits, params, history_dev, n_history, forbid_dev,
                                   n_forbid, stop_ids, n_stop, rng_dev, token_out_dev, done_out_dev, status_out_dev);
    if (rc != QW3_OK) return rc;  // rows beyond QW3_SAMPLE_MAX_ROWS or a vocabulary beyond QW3_SAMPLE_MAX_VOCAB
    if (sample_scratch_bytes(n_rows) > kNoAllocScratchBytes) return QW3_OUT_OF_MEMORY;
    void *ws = nullptr;
    const int32_t src = noalloc_scratch(&ws);
    if (src != QW3_OK) return src;
    sample_bind_scratch(a, ws);
    return launch_sample(a, (hipStream_t)stream) == hipSuccess ? QW3_OK : QW3_DEVICE_ERROR;
}

}  // extern "C"
