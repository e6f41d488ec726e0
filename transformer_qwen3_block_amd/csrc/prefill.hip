// Tiled prefill of bf16-weight models on gfx950 MFMA: RMSNorm rows, Q/K/V GEMM, QK-Norm + RoPE + KV append,
// causal GQA flash attention, o_proj GEMM + residual, RMSNorm rows, gate/up GEMM + SwiGLU, down GEMM +
// residual.  MFMA operands are f16 with f32 accumulation: the packer keeps an f16 copy of each bf16
// projection (bf16 -> f16 is exact for |w| >= 2^-14), activations are rounded to f16 (11-bit significand,
// eight times finer than bf16), and the bf16 K/V cache is widened to f16 while it is staged in LDS.  The
// residual stream stays f32.  An activation beyond the f16 range becomes infinite and reaches the logits,
// where the non-finite check latches a numerical failure; a cached key or value beyond it (the attention's
// f16 shadow of the bf16 cache) latches kStatusF16Range where it is converted, since a key converted to
// infinity could otherwise leave the softmax with a zero weight instead of a non-finite result.
//
// MFMA v_mfma_f32_16x16x32_f16 lane layout (wave64): lane l supplies A[l%16][8*(l/16)+e] and
// B[8*(l/16)+e][l%16] (e = 0..7) and receives C[4*(l/16)+r][l%16] (r = 0..3).
//
// Page titles used in citations:
//   [P1] "Scalar-Native Qwen3 Reference Runtime As The Numerical Authority"
//   [P4] "Portable WebAssembly Runtime Architecture for TinyRustLM"
#include <math.h>

#include <type_traits>

#include "prefill.h"

namespace qw3 {

namespace {

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ f16x8_t as_f16x8(const uint4 &v) { return __builtin_bit_cast(f16x8_t, v); }

__device__ __forceinline__ f32x4_t mfma16(const uint4 &a, const uint4 &b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(a), as_f16x8(b), c, 0, 0, 0);
}

// f32 -> f16 bits, round to nearest even
__device__ __forceinline__ uint16_t f32_to_h16(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }
__device__ __forceinline__ float h16_to_f32(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

// Two f32 -> packed f16 pair, round to nearest even (one packed conversion on gfx950).
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_h16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, f16x2_t));
}

__global__ void bf16_to_f16_kernel(const uint16_t *in, uint16_t *out, size_t n) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) out[i] = f32_to_h16(bf16_to_f32(in[i]));
}

// ---------------------------------------------------------------------------------------------------
// RMSNorm of T rows ([P1] section 2 items 1 and 6), written as f16 MFMA operands.  One wave per row: the
// row stays in registers (H / 64 values per lane, H a multiple of 256), the sum of squares is a wave
// reduction, no workgroup barrier.
// ---------------------------------------------------------------------------------------------------
template <int VPL, int RPW>  // values per lane (H / 64), rows per wave
__global__ __launch_bounds__(256) void rmsnorm_rows_kernel(const float *x, int T, const float *w, float eps,
                                                           uint16_t *out) {
    constexpr int H = 64 * VPL;
    const int t0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW, lane = threadIdx.x & 63;
    if (t0 >= T) return;
    // the wave's rows and the norm weights, all loads in flight before the first reduction
    float4 v[RPW][VPL / 4], wg[VPL / 4];
#pragma unroll
    for (int q = 0; q < RPW; ++q) {
        const float *xr = x + (size_t)min(t0 + q, T - 1) * H;
#pragma unroll
        for (int i = 0; i < VPL / 4; ++i) v[q][i] = *(const float4 *)(xr + 256 * i + 4 * lane);
    }
#pragma unroll
    for (int i = 0; i < VPL / 4; ++i) wg[i] = *(const float4 *)(w + 256 * i + 4 * lane);
#pragma unroll
    for (int q = 0; q < RPW; ++q) {
        const int t = t0 + q;
        if (t >= T) break;
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < VPL / 4; ++i)
            ss += (v[q][i].x * v[q][i].x + v[q][i].y * v[q][i].y) + (v[q][i].z * v[q][i].z + v[q][i].w * v[q][i].w);
        const float inv = 1.0f / sqrtf(wave_sum_fast(ss) / (float)H + eps);
#pragma unroll
        for (int i = 0; i < VPL / 4; ++i) {
            const int k = 256 * i + 4 * lane;
            const float4 g = wg[i];
            ushort4 o;
            o.x = f32_to_h16(g.x * (v[q][i].x * inv));
            o.y = f32_to_h16(g.y * (v[q][i].y * inv));
            o.z = f32_to_h16(g.z * (v[q][i].z * inv));
            o.w = f32_to_h16(g.w * (v[q][i].w * inv));
            *(ushort4 *)(out + (size_t)t * H + k) = o;
        }
    }
}

// Any H (a multiple of 4): one workgroup per row, workgroup reduction.
__global__ __launch_bounds__(256) void rmsnorm_rows_any_kernel(const float *x, int H, const float *w, float eps,
                                                               uint16_t *out) {
    __shared__ float red[4];
    const int t = blockIdx.x, tid = threadIdx.x;
    const float *xr = x + (size_t)t * H;
    float ss = 0.f;
    for (int k = tid * 4; k < H; k += 1024) {
        const float4 v = *(const float4 *)(xr + k);
        ss += (v.x * v.x + v.y * v.y) + (v.z * v.z + v.w * v.w);
    }
    ss = wave_sum(ss);
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    const float inv = 1.0f / sqrtf(((red[0] + red[1]) + (red[2] + red[3])) / (float)H + eps);
    for (int k = tid * 4; k < H; k += 1024) {
        const float4 v = *(const float4 *)(xr + k);
        const float4 g = *(const float4 *)(w + k);
        ushort4 o;
        o.x = f32_to_h16(g.x * (v.x * inv));
        o.y = f32_to_h16(g.y * (v.y * inv));
        o.z = f32_to_h16(g.z * (v.z * inv));
        o.w = f32_to_h16(g.w * (v.w * inv));
        *(ushort4 *)(out + (size_t)t * H + k) = o;
    }
}

hipError_t launch_rmsnorm_rows(const float *x, int T, int H, const float *w, float eps, uint16_t *out,
                               hipStream_t st) {
    constexpr int RPW = 2;  // rows per wave: twice the loads in flight per wave
    const dim3 grid((T + 4 * RPW - 1) / (4 * RPW));
    switch (H) {
        case 512: hipLaunchKernelGGL((rmsnorm_rows_kernel<8, RPW>), grid, dim3(256), 0, st, x, T, w, eps, out); break;
        case 1024: hipLaunchKernelGGL((rmsnorm_rows_kernel<16, RPW>), grid, dim3(256), 0, st, x, T, w, eps, out); break;
        case 2048: hipLaunchKernelGGL((rmsnorm_rows_kernel<32, RPW>), grid, dim3(256), 0, st, x, T, w, eps, out); break;
        default:
            if (H % 4) return hipErrorInvalidValue;
            hipLaunchKernelGGL(rmsnorm_rows_any_kernel, dim3(T), dim3(256), 0, st, x, H, w, eps, out);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------------
// C[M, N] = A[M, K] * W[N, K]^T on f16 MFMA with f32 accumulation.
// Workgroup tile BM x BN; WM x WN waves, each owning a (BM/WM) x (BN/WN) block of 16x16 tiles.  K runs in
// steps of 64 through a ring of S LDS stages filled by direct-to-LDS loads (global_load_lds_dwordx4: each
// wave instruction lands 1 KB, lane l's 16 bytes at byte 16 l, with no registers or LDS store instructions
// on the way): while step j is multiplied, steps j+1 .. j+S-2 are in flight, and each step needs one
// barrier.  A stage holds the A and B tiles as 128-byte rows (64 f16) whose eight 16-byte chunks are stored
// XOR-swizzled (chunk c of row r at slot c ^ (r & 7)), so the eight rows one fragment read touches hit
// eight different bank groups; the swizzle is applied by choosing which global chunk each lane loads.
// Workgroups are mapped
// so that the tiles one XCD runs (workgroup b runs on XCD b mod 8) share their column blocks, which keeps
// their weight rows in that XCD's L2.
// Epilogues: f32 store, f16 store, f32 residual add (in place), or SwiGLU into f16: with GLU, each wave's columns are
// half gate rows and half the matching up rows (up rows start at W row `up_off`), so gate and up of one
// output element meet in the same lane.  Split K (short prompts, whose few tiles would otherwise walk every K
// step on a few compute units): each workgroup stores the f32 partial tile of its K range and
// splitk_reduce_kernel adds the ranges in split order and applies the epilogue.
// ---------------------------------------------------------------------------------------------------
enum GemmEpi { G_STORE = 0, G_RESID = 1, G_SWIGLU = 2, G_STORE16 = 3, G_QKNORM = 4 };

struct GemmArgs {
    const uint16_t *A;  // f16 [M][K]
    const uint16_t *W;  // f16 weight rows [*][K]
    int M, N, K;        // N = columns of C (SwiGLU: 2 x output columns)
    int up_off;         // SwiGLU: first up row of W
    float *outf;        // G_STORE / G_RESID: [M][ldo]
    uint16_t *out16;    // G_SWIGLU / G_STORE16: f16 [M][ldo]
    int ldo;
    // G_QKNORM (the Q/K/V projection of a prefill chunk, columns = HQ query, HKV key, HKV value heads of 128):
    // QK-Norm, RoPE and the KV append straight from the accumulators, as qknorm_rope_append_kernel does
    const float *q_norm, *k_norm, *rope_cos, *rope_sin;
    float eps;
    int HQ, HKV, pos0, max_ctx;
    uint16_t *q16, *kc, *vc;
    // optional (pos0 a multiple of 64): the attention's f16 shadow of K ([HKV][ps][128]) and V^T ([HKV][128][ps]),
    // written for the chunk's positions from the same staged tile; null: left to kv16_convert_kernel
    uint16_t *ks16, *vt16;
    int ps;
    int *status;        // kStatusF16Range is latched when a shadow value overflows the f16 range
    // split K (gemm_split_kernel): the f32 partial tiles of the K ranges
    float *part;
};

__host__ __device__ inline int kv16_stride(int max_ctx) { return (max_ctx + 63) & ~63; }
// key slot of position p inside its 32-key group of the V^T shadow (see kv16_convert_kernel)
__device__ __forceinline__ int vt_perm(int p) {
    const int kk = p & 31;
    return (p & ~31) + 8 * ((kk & 15) >> 2) + 4 * (kk >> 4) + (kk & 3);
}
__device__ __forceinline__ uint32_t bf16x2_to_h16x2(uint32_t w) { return pack_h16x2(bf16_lo(w), bf16_hi(w)); }
// A packed f16 pair holding an infinity or NaN (exponent all ones).  The bf16 cache keeps keys and values beyond
// 65504, their f16 shadow does not: a key there would score +-inf and could silently drop out of the softmax,
// so every shadow write checks its values and latches kStatusF16Range instead.
__device__ __forceinline__ bool h16x2_nonfinite(uint32_t w) {
    return (w & 0x7c00u) == 0x7c00u || (w & 0x7c000000u) == 0x7c000000u;
}

constexpr int kBK = 64;
constexpr int kLdsPad = 16;  // 16-bit elements of padding per LDS row of the split-K kernel's register-staged tiles

// Wait until at most N vector-memory operations of this wave are outstanding and every LDS operation has
// completed (the waitcnt immediate of gfx9: vmcnt in bits 3:0 and 15:14, expcnt 6:4 left at its maximum,
// lgkmcnt 11:8 = 0).
template <int N>
__device__ __forceinline__ void wait_vm_lds() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4));
}
// The wait before step j's barrier: every load of step j done, those of the `ahead` (< D) later steps that
// have been issued may still fly.  Loads of one wave complete in issue order.
template <int LPS, int D>
__device__ __forceinline__ void wait_steps(int ahead) {
    if constexpr (D <= 0) {
        wait_vm_lds<0>();
    } else {
        if (ahead >= D)
            wait_vm_lds<D * LPS>();
        else
            wait_steps<LPS, D - 1>(ahead);
    }
}
// One 16-byte direct-to-LDS load per lane: lane l's bytes land at LDS byte `lds` + 16 l (`lds` is the same
// for the whole wave).  Written as an instruction the compiler does not see into, so that it adds no wait
// for these loads before LDS reads of other stages; the K loop's own waits order them.  The instruction
// has no register results.
__device__ __forceinline__ void lds_dma16(const void *gaddr, const void *lds) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gaddr), "s"(m0) : "memory", "m0");
}

// LDS bytes an epilogue stages after the K loop (the ring is reused)
template <int BM, int BN, int WM, int WN, int EPI>
constexpr int gemm_epi_bytes() {
    return EPI == G_SWIGLU   ? BM * (BN / 2 + 8) * 2
           : EPI == G_RESID  ? BM * (BN + 4) * 4
           : EPI == G_QKNORM ? BM * (BN + 8) * 2 + WM * WN * (8 * 64 + BM / WM) * 4
                             : 0;
}

template <int BM, int BN, int WM, int WN, int EPI, int S>
__global__ __launch_bounds__(64 * WM * WN) void gemm_f16_kernel(GemmArgs g) {
    constexpr int NW = WM * WN, NT = 64 * NW;    // waves, threads
    constexpr int WTM = BM / WM, WTN = BN / WN;  // wave tile
    constexpr int TM = WTM / 16, TN = WTN / 16;
    constexpr int ACH = BM * 8 / NT, BCH = BN * 8 / NT;  // 1 KB load instructions per wave per step (A, B)
    constexpr int LPS = ACH + BCH;
    constexpr int STAGE = (BM + BN) * kBK;  // f16 elements per ring stage
    static_assert(ACH * NT == BM * 8 && BCH * NT == BN * 8 && TM >= 1 && TN >= 1, "tile does not fit the wave layout");
    static_assert(S >= 2 && (S - 2) * LPS < 64, "ring depth");
    constexpr int RING = S * STAGE * 2, EPIB = gemm_epi_bytes<BM, BN, WM, WN, EPI>();
    // one LDS region: the ring of staging tiles, reused by the epilogue
    __shared__ __attribute__((aligned(1024))) uint16_t smem[(RING > EPIB ? RING : EPIB) / 2];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    // XCD-aware tile order: the tiles of one XCD are consecutive in column-major tile order
    const int ntm = (g.M + BM - 1) / BM, nt = ntm * (g.N / BN);
    int tile = blockIdx.x;
    if (nt % 8 == 0) tile = (blockIdx.x & 7) * (nt / 8) + (blockIdx.x >> 3);
    const int m0 = (tile % ntm) * BM, n0 = (tile / ntm) * BN;

    // weight row of tile row r
    auto wrow = [&](int r) -> long long {
        if constexpr (EPI == G_SWIGLU) {
            const int wv = r / WTN, q = r % WTN, half = WTN / 2;
            const int col = n0 / 2 + wv * half + (q % half);
            return q < half ? (long long)col : (long long)g.up_off + col;
        } else {
            return (long long)n0 + r;
        }
    };

    // Load instruction c of this wave covers tile rows 8 (c NW + wave) .. +7; lane l fetches the chunk stored
    // at slot l & 7 of row l >> 3 there, i.e. logical chunk (l & 7) ^ (row & 7).  Rows past M read row M-1
    // (the epilogue drops their products).  Addresses are formed once; a step adds its column offset.
    const uint16_t *pa[ACH];
    const uint16_t *pb[BCH];
#pragma unroll
    for (int c = 0; c < ACH; ++c) {
        const int ch = (c * NW + wave) * 64 + lane, r = ch >> 3, lc = (ch & 7) ^ (r & 7);
        pa[c] = g.A + (size_t)min(m0 + r, g.M - 1) * g.K + lc * 8;
    }
#pragma unroll
    for (int c = 0; c < BCH; ++c) {
        const int ch = (c * NW + wave) * 64 + lane, r = ch >> 3, lc = (ch & 7) ^ (r & 7);
        pb[c] = g.W + (size_t)wrow(r) * g.K + lc * 8;
    }
    const int nsteps = g.K / kBK;
    auto issue = [&](int step) {
        const int k0 = step * kBK;
        uint16_t *sa = smem + (step % S) * STAGE, *sb = sa + BM * kBK;
#pragma unroll
        for (int c = 0; c < ACH; ++c) lds_dma16(pa[c] + k0, sa + (c * NW + wave) * 512);
#pragma unroll
        for (int c = 0; c < BCH; ++c) lds_dma16(pb[c] + k0, sb + (c * NW + wave) * 512);
    };

    f32x4_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int jj = 0; jj < TN; ++jj) acc[i][jj] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // fragment reads: lane (row lrow of a 16-row block, column group lq) takes logical chunk 4 kk + lq of its
    // row, stored at slot (4 kk + lq) ^ (lrow & 7) (block bases are multiples of 8 rows)
    const int lrow = lane & 15, lq = lane >> 4, sw = lane & 7;
    auto multiply = [&](int step) {
        const uint16_t *as = smem + (step % S) * STAGE, *bs = as + BM * kBK;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int slot = ((4 * kk + lq) ^ sw) * 8;
            uint4 af[TM], bfr[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) af[i] = *(const uint4 *)(as + (wm * WTM + i * 16 + lrow) * kBK + slot);
#pragma unroll
            for (int jj = 0; jj < TN; ++jj) bfr[jj] = *(const uint4 *)(bs + (wn * WTN + jj * 16 + lrow) * kBK + slot);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int jj = 0; jj < TN; ++jj) acc[i][jj] = mfma16(af[i], bfr[jj], acc[i][jj]);
        }
    };

#pragma unroll
    for (int st = 0; st < S - 1; ++st)
        if (st < nsteps) issue(st);
    for (int j = 0; j < nsteps; ++j) {
        // this wave's loads of step j have landed and its reads of step j-1 are done; after the barrier the
        // same holds for every wave, so step j is complete in LDS and stage (j-1) mod S may be refilled
        wait_steps<LPS, S - 2>(nsteps - 1 - j);
        asm volatile("s_barrier" ::: "memory");
        if (j + S - 1 < nsteps) issue(j + S - 1);
        multiply(j);
    }
    __syncthreads();  // every wave's last reads done before an epilogue reuses the ring (no loads in flight)

    // epilogue: lane holds C[4*(lane/16) + r][lane%16] of each 16x16 tile
    const int crow = 4 * (lane >> 4), ccol = lane & 15;
    if constexpr (EPI == G_SWIGLU && BM * (BN / 2 + 8) * 2 <= (int)sizeof(smem)) {
        // SwiGLU, [P1] section 5: (g * sigmoid(g)) * u, staged as an f16 tile in LDS (the staging region is
        // free after the K loop's last barrier) and written in 16-byte chunks covering whole row segments
        constexpr int OCW = BN / 2, OLD = OCW + 8;  // output columns of the tile, f16 per staged row
        uint16_t *ot = smem;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int jj = 0; jj < TN / 2; ++jj) {
                    const float gt = acc[i][jj][r], up = acc[i][jj + TN / 2][r];
                    const float sig = 1.0f / (1.0f + __expf(-gt));
                    ot[(wm * WTM + i * 16 + crow + r) * OLD + wn * (WTN / 2) + jj * 16 + ccol] = f32_to_h16((gt * sig) * up);
                }
        __syncthreads();
        for (int c = tid; c < BM * (OCW / 8); c += NT) {
            const int row = c / (OCW / 8), c8 = (c % (OCW / 8)) * 8, m = m0 + row;
            if (m >= g.M) continue;
            *(uint4 *)(g.out16 + (size_t)m * g.ldo + n0 / 2 + c8) = *(const uint4 *)(ot + row * OLD + c8);
        }
        return;
    }
    if constexpr (EPI == G_RESID && BM * (BN + 4) * 4 <= (int)sizeof(smem)) {
        // residual add through an LDS copy of the tile (the staging region is free: the K loop ended with a
        // barrier), so the read-modify-write of x runs in 16-byte chunks covering whole row segments
        constexpr int CLD = BN + 4;  // floats per staged row
        float *ct = (float *)smem;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int jj = 0; jj < TN; ++jj)
                    ct[(wm * WTM + i * 16 + crow + r) * CLD + wn * WTN + jj * 16 + ccol] = acc[i][jj][r];
        __syncthreads();
        for (int c = tid; c < BM * (BN / 4); c += NT) {
            const int row = c / (BN / 4), c4 = (c % (BN / 4)) * 4, m = m0 + row;
            if (m >= g.M) continue;
            float4 *px = (float4 *)(g.outf + (size_t)m * g.ldo + n0 + c4);
            const float4 a4 = *(const float4 *)(ct + row * CLD + c4);
            float4 x4 = *px;
            x4.x += a4.x;
            x4.y += a4.y;
            x4.z += a4.z;
            x4.w += a4.w;
            *px = x4;
        }
        return;
    }
    if constexpr (EPI == G_QKNORM) {
        // A head's 128 columns are the 64-column tiles of waves wn and wn ^ 1 (same wm); the per-row sums of
        // squares and the RoPE partner halves (dims d and d + 64) cross between the two through LDS, 8 rows per
        // wave at a time; results are staged as a 2-byte tile in LDS and leave in 16-byte chunks.  All of it in
        // the staging region, free after the K loop (which ends with a barrier).  [P1] section 2 items 3-4 and
        // the section 6 append: the same steps and rounding points as qknorm_rope_append_kernel, from the f32
        // accumulators.
        constexpr int OLD = BN + 8;  // 2-byte elements per staged output row (16-byte padding)
        static_assert(WTN == 64 && WN % 2 == 0 && BN % 128 == 0 && TM * 16 == WTM, "a head spans two waves' 64 columns");
        static_assert(BM * OLD * 2 + (WM * WN * (8 * 64 + WTM)) * 4 <= (int)sizeof(smem), "epilogue fits in LDS");
        uint16_t *otile = smem;                        // [BM][OLD]
        float *xch = (float *)(smem + BM * OLD);       // [wave][8 rows][64]
        float *ssq = xch + WM * WN * 8 * 64;           // [wave][WTM]
        const int partner = wave ^ 1;
        const int hcol = (n0 + wn * WTN) / kHeadDim;  // this wave's head among the Q/K/V heads
        const bool is_q = hcol < g.HQ, is_v = hcol >= g.HQ + g.HKV;
        const int dlo = (wn & 1) * 64;              // the wave's dims within its head
        float wv[TN];
#pragma unroll
        for (int jj = 0; jj < TN; ++jj) wv[jj] = is_v ? 1.f : (is_q ? g.q_norm : g.k_norm)[dlo + jj * 16 + ccol];
        if (!is_v) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float p = 0.f;
#pragma unroll
                    for (int jj = 0; jj < TN; ++jj) p += acc[i][jj][r] * acc[i][jj][r];
                    p = row16_sum(p);  // the 16 lanes of a row group hold the wave's 64 columns
                    if (ccol == 0) ssq[wave * WTM + i * 16 + crow + r] = p;
                }
        }
        const float qs = (1.0f / sqrtf((float)kHeadDim)) * kLog2e;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int rh = 0; rh < 2; ++rh) {
                // this pass: rows crow + 2 rh + q (q = 0, 1) of sub-tile i; its RoPE table entries first
                float cs[2][TN], sn[2][TN];
                if (!is_v) {
#pragma unroll
                    for (int q = 0; q < 2; ++q) {
                        const int m = m0 + wm * WTM + i * 16 + crow + 2 * rh + q;
                        const size_t pr = (size_t)(g.pos0 + (m < g.M ? m : 0)) * 64;
#pragma unroll
                        for (int jj = 0; jj < TN; ++jj) {
                            cs[q][jj] = g.rope_cos[pr + jj * 16 + ccol];
                            sn[q][jj] = g.rope_sin[pr + jj * 16 + ccol];
                        }
                    }
                }
                __syncthreads();  // ssq complete (first pass) / the previous pass's exchange has been read
                float nv[2][TN];
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const int rl = i * 16 + crow + 2 * rh + q;
                    const float inv =
                        is_v ? 1.f
                             : 1.0f / sqrtf((ssq[wave * WTM + rl] + ssq[partner * WTM + rl]) / (float)kHeadDim + g.eps);
#pragma unroll
                    for (int jj = 0; jj < TN; ++jj) {
                        nv[q][jj] = is_v ? acc[i][jj][2 * rh + q] : wv[jj] * (acc[i][jj][2 * rh + q] * inv);
                        xch[(wave * 8 + 2 * (lane >> 4) + q) * 64 + jj * 16 + ccol] = nv[q][jj];
                    }
                }
                __syncthreads();
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const int orow = wm * WTM + i * 16 + crow + 2 * rh + q;
#pragma unroll
                    for (int jj = 0; jj < TN; ++jj) {
                        float o = nv[q][jj];
                        if (!is_v) {
                            const float other = xch[(partner * 8 + 2 * (lane >> 4) + q) * 64 + jj * 16 + ccol];
                            o = dlo == 0 ? o * cs[q][jj] - other * sn[q][jj] : o * cs[q][jj] + other * sn[q][jj];
                        }
                        otile[orow * OLD + wn * WTN + jj * 16 + ccol] = is_q ? f32_to_h16(o * qs) : f32_to_bf16(o);
                    }
                }
            }
        }
        __syncthreads();
        // the staged tile out in 16-byte chunks: query heads to q16, key and value heads into the cache
        constexpr int CPR = BN / 8;
        for (int c = tid; c < BM * CPR; c += NT) {
            const int row = c / CPR, cc = (c % CPR) * 8, m = m0 + row;
            if (m >= g.M) continue;
            const int col = n0 + cc, h = col / kHeadDim, d = col % kHeadDim;
            uint16_t *dst = h < g.HQ ? g.q16 + ((size_t)m * g.HQ + h) * kHeadDim + d
                            : h < g.HQ + g.HKV
                                ? g.kc + ((size_t)(h - g.HQ) * g.max_ctx + g.pos0 + m) * kHeadDim + d
                                : g.vc + ((size_t)(h - g.HQ - g.HKV) * g.max_ctx + g.pos0 + m) * kHeadDim + d;
            const uint4 v = *(const uint4 *)(otile + row * OLD + cc);
            *(uint4 *)dst = v;
            if (g.ks16 && h >= g.HQ && h < g.HQ + g.HKV) {  // the key row's f16 shadow (exact: bf16 values in range)
                const uint4 hv =
                    make_uint4(bf16x2_to_h16x2(v.x), bf16x2_to_h16x2(v.y), bf16x2_to_h16x2(v.z), bf16x2_to_h16x2(v.w));
                *(uint4 *)(g.ks16 + ((size_t)(h - g.HQ) * g.ps + g.pos0 + m) * kHeadDim + d) = hv;
                if (h16x2_nonfinite(hv.x) || h16x2_nonfinite(hv.y) || h16x2_nonfinite(hv.z) || h16x2_nonfinite(hv.w))
                    atomicOr(g.status, kStatusF16Range);
            }
        }
        // V^T shadow of the tile's value heads: 16-byte chunks of 8 key slots of a 32-position group (the
        // tile's rows start at a multiple of 64 positions); rows past the chunk's last position up to the next
        // multiple of 64 get zero, so every attention tile holds finite values
        if (g.ks16 && (n0 + BN) / kHeadDim > g.HQ + g.HKV) {
            const int vrows = min(BM, ((g.M - m0) + 63) & ~63);  // rows of this tile the shadow covers
            constexpr int SG = BM / 8;                           // 8-slot groups per dim of a full tile
            for (int c = tid; c < (BN / kHeadDim) * kHeadDim * SG; c += NT) {
                const int hl = c / (kHeadDim * SG), dim = (c / SG) % kHeadDim, sg = c % SG;  // powers of two
                const int h = n0 / kHeadDim + hl;
                if (h < g.HQ + g.HKV || 8 * sg >= vrows) continue;  // query / key head of a mixed tile, or past the rows
                uint32_t pk[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float f2[2];
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const int s8 = 8 * (sg & 3) + 2 * e + u;  // slot within the 32-group
                        const int row = 32 * (sg >> 2) + 16 * ((s8 >> 2) & 1) + 4 * (s8 >> 3) + (s8 & 3);
                        f2[u] = m0 + row < g.M ? bf16_to_f32(otile[row * OLD + hl * kHeadDim + dim]) : 0.f;
                    }
                    pk[e] = pack_h16x2(f2[0], f2[1]);
                }
                if (h16x2_nonfinite(pk[0]) || h16x2_nonfinite(pk[1]) || h16x2_nonfinite(pk[2]) || h16x2_nonfinite(pk[3]))
                    atomicOr(g.status, kStatusF16Range);
                *(uint4 *)(g.vt16 + ((size_t)(h - g.HQ - g.HKV) * kHeadDim + dim) * g.ps + g.pos0 + m0 + 8 * sg) =
                    make_uint4(pk[0], pk[1], pk[2], pk[3]);
            }
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = m0 + wm * WTM + i * 16 + crow + r;
            if (m >= g.M) continue;
            if constexpr (EPI == G_SWIGLU) {
#pragma unroll
                for (int jj = 0; jj < TN / 2; ++jj) {
                    const int col = n0 / 2 + wn * (WTN / 2) + jj * 16 + ccol;
                    const float gt = acc[i][jj][r], up = acc[i][jj + TN / 2][r];
                    // SwiGLU, [P1] section 5: (g * sigmoid(g)) * u
                    const float sig = 1.0f / (1.0f + __expf(-gt));
                    g.out16[(size_t)m * g.ldo + col] = f32_to_h16((gt * sig) * up);
                }
            } else if constexpr (EPI == G_STORE16) {
#pragma unroll
                for (int jj = 0; jj < TN; ++jj)
                    g.out16[(size_t)m * g.ldo + n0 + wn * WTN + jj * 16 + ccol] = f32_to_h16(acc[i][jj][r]);
            } else {
#pragma unroll
                for (int jj = 0; jj < TN; ++jj) {
                    const int n = n0 + wn * WTN + jj * 16 + ccol;
                    float *p = g.outf + (size_t)m * g.ldo + n;
                    if constexpr (EPI == G_STORE)
                        *p = acc[i][jj][r];
                    else
                        *p = *p + acc[i][jj][r];
                }
            }
        }
    }
}

template <int BM, int BN, int WM, int WN, int EPI, int S>
hipError_t launch_gemm_cfg(const GemmArgs &g, hipStream_t st) {
    if (g.K % kBK || g.N % BN || g.M < 1) return hipErrorInvalidValue;
    const int nt = ((g.M + BM - 1) / BM) * (g.N / BN);
    hipLaunchKernelGGL((gemm_f16_kernel<BM, BN, WM, WN, EPI, S>), dim3(nt), dim3(64 * WM * WN), 0, st, g);
    return hipGetLastError();
}

// Tile shapes and ring depths measured fastest on the 2048-token shapes with the weights streaming from HBM
// (Q/K/V 4096 x 1024, gate/up 6144 x 1024, o_proj 1024 x 2048, down 1024 x 3072).
template <int EPI>
hipError_t launch_gemm(const GemmArgs &g, hipStream_t st) {
    if (g.K % (2 * kBK) || g.N % 128) return hipErrorInvalidValue;
    if constexpr (EPI == G_QKNORM) {  // tiles whose waves hold 64 columns: two waves per 128-column head
        if (g.M <= 64) return hipErrorInvalidValue;
        if (g.N % 256 == 0 && ((g.M + 127) / 128) * (g.N / 256) >= 256)
            return launch_gemm_cfg<128, 256, 4, 4, EPI, 3>(g, st);
        return launch_gemm_cfg<128, 128, 4, 2, EPI, 2>(g, st);
    } else {
        if (g.M <= 64) return launch_gemm_cfg<64, 32, 4, 1, EPI, 3>(g, st);  // short prompts: weight-streaming bound
        if (EPI != G_SWIGLU && g.N <= 1024) return launch_gemm_cfg<128, 64, 4, 2, EPI, 4>(g, st);  // narrow outputs
        if constexpr (EPI == G_SWIGLU)
            if (g.M > 512 && g.N % 256 == 0) return launch_gemm_cfg<256, 256, 4, 4, EPI, 2>(g, st);
        if ((EPI == G_STORE || EPI == G_STORE16) && g.N % 256 == 0 && ((g.M + 127) / 128) * (g.N / 256) >= 256)
            return launch_gemm_cfg<128, 256, 4, 4, EPI, 3>(g, st);
        return launch_gemm_cfg<128, 128, 4, 2, EPI, 2>(g, st);
    }
}

// Split-K products for prompts of up to kSplitMaxT tokens: 64 x 64 tiles, K split so that about kSplitWg
// workgroups run (each range an even number of 64-column steps); the partial tiles stay within
// kSplitScratchFloats.  Reduction: output element (m, n) adds its ranges' partials in split order, then the
// epilogue of the unsplit product (residual add, f16 store, or SwiGLU of gate column u and up column up_off + u).
constexpr int kSplitBM = 64, kSplitBN = 64;
constexpr int kSplitWg = 1024;  // split tiles at most (kSplitScratchFloats / (64 x 64))
constexpr int kSplitMax = 16;   // K ranges at most
constexpr int kSplitSteps = 8;  // K steps per range at most (all in flight in registers)
static_assert((uint64_t)kSplitWg * kSplitBM * kSplitBN <= kSplitScratchFloats, "partial tiles fit the scratch");

// One 64 x 64 tile over KS steps of 64 columns (K range split * KS .. split * KS + KS - 1, split = blockIdx.y),
// for prompts too short for the K loop of gemm_f16_kernel to hide its load latency: every step's loads are
// issued at once, then the steps go through two LDS buffers (one barrier each) into the MFMA accumulators.
// Four waves of 32 x 32; the f32 tile is stored whole to part[(split * tiles + tile) * 64 * 64 + row * 64 + col].
template <int KS>
__global__ __launch_bounds__(256) void gemm_split_kernel(GemmArgs g) {
    constexpr int BM = kSplitBM, BN = kSplitBN, WN = 2, WTM = 32, WTN = 32, TM = 2, TN = 2;
    constexpr int LDR = kBK + kLdsPad, NT = 256;
    constexpr int ACH = BM * kBK / 8 / NT, BCH = BN * kBK / 8 / NT;
    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (BM + BN) * LDR];
    uint16_t(*As)[BM * LDR] = reinterpret_cast<uint16_t(*)[BM * LDR]>(smem);
    uint16_t(*Bs)[BN * LDR] = reinterpret_cast<uint16_t(*)[BN * LDR]>(smem + 2 * BM * LDR);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave / WN, wn = wave % WN;
    const int ntm = (g.M + BM - 1) / BM, nt = ntm * (g.N / BN);
    int tile = blockIdx.x;
    if (nt % 8 == 0) tile = (blockIdx.x & 7) * (nt / 8) + (blockIdx.x >> 3);
    const int m0 = (tile % ntm) * BM, n0 = (tile / ntm) * BN;
    const int kbase = (int)blockIdx.y * KS * kBK;
    uint4 ra[KS][ACH], rb[KS][BCH];
    int la[ACH], lb[BCH];
#pragma unroll
    for (int c = 0; c < ACH; ++c) {
        const int ch = tid + NT * c, r = ch >> 3, kc = (ch & 7) * 8;
        const uint16_t *pa = g.A + (size_t)min(m0 + r, g.M - 1) * g.K + kbase + kc;  // rows past M: row M-1
        la[c] = r * LDR + kc;
#pragma unroll
        for (int st = 0; st < KS; ++st) {
            const u32x4_t v = *(const u32x4_t *)(pa + st * kBK);
            ra[st][c] = make_uint4(v.x, v.y, v.z, v.w);
        }
    }
#pragma unroll
    for (int c = 0; c < BCH; ++c) {
        const int ch = tid + NT * c, r = ch >> 3, kc = (ch & 7) * 8;
        const uint16_t *pb = g.W + (size_t)(n0 + r) * g.K + kbase + kc;
        lb[c] = r * LDR + kc;
#pragma unroll
        for (int st = 0; st < KS; ++st) rb[st][c] = load_nt16(pb + st * kBK);
    }
    f32x4_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int jj = 0; jj < TN; ++jj) acc[i][jj] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int ksub = 8 * (lane >> 4), lrow = lane & 15;
#pragma unroll
    for (int st = 0; st < KS; ++st) {
        // buffer st & 1 was last read by step st - 2, which every wave finished before step st - 1's barrier
        uint16_t *as = As[st & 1], *bs = Bs[st & 1];
#pragma unroll
        for (int c = 0; c < ACH; ++c) *(uint4 *)(as + la[c]) = ra[st][c];
#pragma unroll
        for (int c = 0; c < BCH; ++c) *(uint4 *)(bs + lb[c]) = rb[st][c];
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < kBK; kk += 32) {
            uint4 af[TM], bfr[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) af[i] = *(const uint4 *)(as + (wm * WTM + i * 16 + lrow) * LDR + kk + ksub);
#pragma unroll
            for (int jj = 0; jj < TN; ++jj) bfr[jj] = *(const uint4 *)(bs + (wn * WTN + jj * 16 + lrow) * LDR + kk + ksub);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int jj = 0; jj < TN; ++jj) acc[i][jj] = mfma16(af[i], bfr[jj], acc[i][jj]);
        }
    }
    // lane holds C[4*(lane/16) + r][lane%16] of each 16x16 tile; rows past M are stored too (never read)
    const int crow = 4 * (lane >> 4), ccol = lane & 15;
    float *pt = g.part + ((size_t)blockIdx.y * nt + tile) * (BM * BN);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int jj = 0; jj < TN; ++jj)
                pt[(wm * WTM + i * 16 + crow + r) * BN + wn * WTN + jj * 16 + ccol] = acc[i][jj][r];
}

template <int EPI>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmArgs g, int nsplit, int ntm, int nout) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;  // group of 4 output columns
    const int gpr = nout / 4;
    if (i >= (long long)g.M * gpr) return;
    const int m = (int)(i / gpr), c4 = (int)(i % gpr) * 4;
    const int nt = ntm * (g.N / kSplitBN);
    auto sum4 = [&](int n) {  // columns n..n+3 of row m, summed over the splits in order
        const int t = (m / kSplitBM) + ntm * (n / kSplitBN);
        const size_t off = (size_t)t * (kSplitBM * kSplitBN) + (m % kSplitBM) * kSplitBN + (n % kSplitBN);
        const size_t sstride = (size_t)nt * (kSplitBM * kSplitBN);
        float4 s = *(const float4 *)(g.part + off);
        // loads of up to kSplitMax ranges in flight together; the additions keep the split order
        float4 v[kSplitMax - 1];
#pragma unroll
        for (int k = 1; k < kSplitMax; ++k)
            if (k < nsplit) v[k - 1] = *(const float4 *)(g.part + k * sstride + off);
#pragma unroll
        for (int k = 1; k < kSplitMax; ++k)
            if (k < nsplit) {
                s.x += v[k - 1].x;
                s.y += v[k - 1].y;
                s.z += v[k - 1].z;
                s.w += v[k - 1].w;
            }
        return s;
    };
    if constexpr (EPI == G_RESID) {
        float4 *p = (float4 *)(g.outf + (size_t)m * g.ldo + c4);
        const float4 s = sum4(c4), x = *p;
        *p = make_float4(x.x + s.x, x.y + s.y, x.z + s.z, x.w + s.w);
    } else if constexpr (EPI == G_STORE16) {
        const float4 s = sum4(c4);
        uint16_t *o = g.out16 + (size_t)m * g.ldo + c4;
        *(uint2 *)o = make_uint2(pack_h16x2(s.x, s.y), pack_h16x2(s.z, s.w));
    } else {
        static_assert(EPI == G_SWIGLU, "residual, f16 store or SwiGLU");
        const float4 gt = sum4(c4), up = sum4(g.up_off + c4);
        const float gv[4] = {gt.x, gt.y, gt.z, gt.w}, uv[4] = {up.x, up.y, up.z, up.w};
        float a[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            // SwiGLU, [P1] section 5: (g * sigmoid(g)) * u, as the unsplit epilogue computes it
            const float sig = 1.0f / (1.0f + __expf(-gv[e]));
            a[e] = (gv[e] * sig) * uv[e];
        }
        uint16_t *o = g.out16 + (size_t)m * g.ldo + c4;
        *(uint2 *)o = make_uint2(pack_h16x2(a[0], a[1]), pack_h16x2(a[2], a[3]));
    }
}

// Residual products of a short prompt whose output feeds an RMSNorm (o_proj -> the MLP norm, down -> the next
// layer's attention norm): one workgroup per row, each thread a group of four columns per 1024, adds the K
// ranges' partials to the row in split order (as splitk_reduce_kernel<G_RESID>), writes the row back and, with
// nw, normalises it into the f16 operand of the next product (the same arithmetic as rmsnorm_rows_kernel,
// sum of squares by wave then by workgroup): one launch instead of two.
template <int GPT>  // column groups of four per thread (H = 1024 GPT)
__global__ __launch_bounds__(256) void splitk_resid_norm_kernel(GemmArgs g, int nsplit, int ntm, const float *nw,
                                                                float eps, uint16_t *out16) {
    constexpr int H = 1024 * GPT;
    __shared__ float red[4];
    const int m = blockIdx.x, tid = threadIdx.x;
    const size_t sstride = (size_t)ntm * (H / kSplitBN) * (kSplitBM * kSplitBN);
    float4 xv[GPT];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < GPT; ++i) {
        const int n = 1024 * i + 4 * tid;
        const int t = m / kSplitBM + ntm * (n / kSplitBN);
        const size_t off = (size_t)t * (kSplitBM * kSplitBN) + (m % kSplitBM) * kSplitBN + (n % kSplitBN);
        float4 sm = *(const float4 *)(g.part + off);
        float4 v[kSplitMax - 1];
#pragma unroll
        for (int k = 1; k < kSplitMax; ++k)
            if (k < nsplit) v[k - 1] = *(const float4 *)(g.part + k * sstride + off);
#pragma unroll
        for (int k = 1; k < kSplitMax; ++k)
            if (k < nsplit) {
                sm.x += v[k - 1].x;
                sm.y += v[k - 1].y;
                sm.z += v[k - 1].z;
                sm.w += v[k - 1].w;
            }
        float4 *px = (float4 *)(g.outf + (size_t)m * g.ldo + n);
        const float4 x0 = *px;
        const float4 x = make_float4(x0.x + sm.x, x0.y + sm.y, x0.z + sm.z, x0.w + sm.w);
        *px = x;
        xv[i] = x;
        ss += (x.x * x.x + x.y * x.y) + (x.z * x.z + x.w * x.w);
    }
    if (!nw) return;
    ss = wave_sum(ss);
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    const float inv = 1.0f / sqrtf(((red[0] + red[1]) + (red[2] + red[3])) / (float)H + eps);
#pragma unroll
    for (int i = 0; i < GPT; ++i) {
        const int k = 1024 * i + 4 * tid;
        const float4 w = *(const float4 *)(nw + k);
        ushort4 o;
        o.x = f32_to_h16(w.x * (xv[i].x * inv));
        o.y = f32_to_h16(w.y * (xv[i].y * inv));
        o.z = f32_to_h16(w.z * (xv[i].z * inv));
        o.w = f32_to_h16(w.w * (xv[i].w * inv));
        *(ushort4 *)(out16 + (size_t)m * H + k) = o;
    }
}

// Splits of K for g (1: the product is left unsplit): the fewest ranges of at most kSplitSteps steps that give
// at least 256 workgroups, within kSplitWg split tiles.
int splitk_count(const GemmArgs &g) {
    if (g.N % kSplitBN || g.K % kBK) return 1;
    const int nt = ((g.M + kSplitBM - 1) / kSplitBM) * (g.N / kSplitBN), steps = g.K / kBK;
    int best = 1;
    for (int s = 2; s <= kSplitMax && s <= steps; ++s) {
        if (steps % s || steps / s > kSplitSteps || (long long)nt * s > kSplitWg) continue;
        best = s;
        if ((long long)nt * s >= 256) break;
    }
    return best;
}

// EPI: the unsplit product's epilogue (G_RESID, G_STORE16 or G_SWIGLU, the latter over N = 2 x up_off plain
// rows: gate rows 0..up_off-1, up rows up_off..).  g.part must hold nsplit x tiles x 64 x 64 floats.
hipError_t launch_split_partials(const GemmArgs &g, int nsplit, hipStream_t st) {
    const int ntm = (g.M + kSplitBM - 1) / kSplitBM, nt = ntm * (g.N / kSplitBN);
    if (nsplit < 2 || nsplit > kSplitMax || g.K % (kBK * nsplit) || g.N % kSplitBN || (long long)nt * nsplit > kSplitWg)
        return hipErrorInvalidValue;
    const int ks = g.K / kBK / nsplit;
    const dim3 grid(nt, nsplit);
    switch (ks) {
        case 1: hipLaunchKernelGGL(gemm_split_kernel<1>, grid, dim3(256), 0, st, g); break;
        case 2: hipLaunchKernelGGL(gemm_split_kernel<2>, grid, dim3(256), 0, st, g); break;
        case 3: hipLaunchKernelGGL(gemm_split_kernel<3>, grid, dim3(256), 0, st, g); break;
        case 4: hipLaunchKernelGGL(gemm_split_kernel<4>, grid, dim3(256), 0, st, g); break;
        case 5: hipLaunchKernelGGL(gemm_split_kernel<5>, grid, dim3(256), 0, st, g); break;
        case 6: hipLaunchKernelGGL(gemm_split_kernel<6>, grid, dim3(256), 0, st, g); break;
        case 7: hipLaunchKernelGGL(gemm_split_kernel<7>, grid, dim3(256), 0, st, g); break;
        case 8: hipLaunchKernelGGL(gemm_split_kernel<8>, grid, dim3(256), 0, st, g); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int EPI>
hipError_t launch_gemm_split(GemmArgs g, int nsplit, hipStream_t st) {
    const hipError_t e = launch_split_partials(g, nsplit, st);
    if (e != hipSuccess) return e;
    const int ntm = (g.M + kSplitBM - 1) / kSplitBM;
    const int nout = EPI == G_SWIGLU ? g.up_off : g.N;
    const long long groups = (long long)g.M * (nout / 4);
    hipLaunchKernelGGL((splitk_reduce_kernel<EPI>), dim3((unsigned)((groups + 255) / 256)), dim3(256), 0, st, g, nsplit, ntm,
                       nout);
    return hipGetLastError();
}

// Split residual product + the RMSNorm of its output (nw null: the residual add only).  g.N = g.ldo = H.
hipError_t launch_split_resid_norm(GemmArgs g, int nsplit, const float *nw, float eps, uint16_t *out16,
                                   hipStream_t st) {
    if (g.ldo != g.N) return hipErrorInvalidValue;
    const hipError_t e = launch_split_partials(g, nsplit, st);
    if (e != hipSuccess) return e;
    const int ntm = (g.M + kSplitBM - 1) / kSplitBM;
    const dim3 grid(g.M);
    switch (g.N) {
        case 1024: hipLaunchKernelGGL((splitk_resid_norm_kernel<1>), grid, dim3(256), 0, st, g, nsplit, ntm, nw, eps, out16); break;
        case 2048: hipLaunchKernelGGL((splitk_resid_norm_kernel<2>), grid, dim3(256), 0, st, g, nsplit, ntm, nw, eps, out16); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------------
// f16 shadow of one layer's K/V for the prefill attention, converted from the bf16 cache after the append:
// K as [kv head][position][128] and V transposed, [kv head][128][position], with the positions of each
// 32-key group ordered so that the keys {4g..4g+3, 16+4g..16+4g+3} sit side by side (one 16-byte read gives
// a lane the eight keys of its P^T fragment).  Positions are padded to a multiple of 64 so every 64-key
// tile is in bounds; the buffer is zeroed at load, so padding and not-yet-written positions hold finite
// values (their attention weights are 0).  The values are f16(bf16 cache value), exact in the f16 range.
// ---------------------------------------------------------------------------------------------------

// Cache positions [0, n) of every KV head into the shadow, 64 positions and a quarter of the head's dims per
// workgroup (grid: position tiles, KV heads, 4): K rows are converted in place of their layout, V goes through
// LDS to be written as 128-byte V^T rows.  Positions past n in the last tile get zero V.
__global__ __launch_bounds__(256) void kv16_convert_kernel(const uint16_t *kc, const uint16_t *vc, int max_ctx,
                                                           int n, uint16_t *ks16, uint16_t *vt16, int *status) {
    constexpr int DQ = kHeadDim / 4;  // dims per workgroup
    __shared__ __attribute__((aligned(16))) uint16_t t[DQ][64 + 8];
    const int p0 = blockIdx.x * 64, hk = blockIdx.y, dq0 = blockIdx.z * DQ, tid = threadIdx.x;
    const int ps = kv16_stride(max_ctx);
    {
        const int c = tid;  // 64 keys x 4 chunks of 8 dims
        const int key = c >> 2, d8 = dq0 + (c & 3) * 8, p = p0 + key;
        uint32_t kw[4] = {0, 0, 0, 0}, vw[4] = {0, 0, 0, 0};
        if (p < n) {
            const size_t at = ((size_t)hk * max_ctx + p) * kHeadDim + d8;
            const uint4 k = *(const uint4 *)(kc + at), v = *(const uint4 *)(vc + at);
            const uint32_t kr[4] = {k.x, k.y, k.z, k.w}, vr[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                kw[e] = pack_h16x2(bf16_lo(kr[e]), bf16_hi(kr[e]));
                vw[e] = pack_h16x2(bf16_lo(vr[e]), bf16_hi(vr[e]));
            }
            bool bad = false;
#pragma unroll
            for (int e = 0; e < 4; ++e) bad = bad || h16x2_nonfinite(kw[e]) || h16x2_nonfinite(vw[e]);
            if (bad) atomicOr(status, kStatusF16Range);
            *(uint4 *)(ks16 + ((size_t)hk * ps + p) * kHeadDim + d8) = make_uint4(kw[0], kw[1], kw[2], kw[3]);
        }
        const int pp = vt_perm(key), dl = d8 - dq0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            t[dl + 2 * e][pp] = (uint16_t)(vw[e] & 0xffffu);
            t[dl + 2 * e + 1][pp] = (uint16_t)(vw[e] >> 16);
        }
    }
    __syncthreads();
    {
        const int c = tid;  // DQ rows x 8 chunks of 8 keys
        const int dim = c >> 3, k8 = (c & 7) * 8;
        *(uint4 *)(vt16 + ((size_t)hk * kHeadDim + dq0 + dim) * ps + p0 + k8) = *(const uint4 *)&t[dim][k8];
    }
}

// ---------------------------------------------------------------------------------------------------
// QK-Norm + RoPE of every query/key head of T tokens ([P1] section 2 items 3-4) and the KV append
// ([P1] section 6), from the f16 Q/K/V projections (the GEMM's f16 epilogue): query heads go to q16 (f16, [T][HQ][128], scaled for the attention kernel); keys (normalised, rotated) and values are
// rounded to bf16 into the cache at positions pos0..pos0+T-1.  One workgroup per token, one wave per head
// at a time; lane i holds dims i and i+64, which is exactly a RoPE pair.
// ---------------------------------------------------------------------------------------------------
constexpr int kQkMaxHeadsPerWave = 8;  // query + key heads of a wave whose loads are in flight together

// SPLIT: the projection ran with K split (gemm_split_kernel) into at most kQkMaxSplit ranges; each element is the
// sum of its ranges' partial tiles in split order, rounded to f16 as the unsplit product's f16 epilogue would.
constexpr int kQkMaxSplit = 4;
template <bool SPLIT>
__global__ __launch_bounds__(256) void qknorm_rope_append_kernel(const uint16_t *qkv, int ldqkv, int HQ, int HKV,
                                                                 const float *q_norm, const float *k_norm,
                                                                 const float *rope_cos, const float *rope_sin,
                                                                 int pos0, float eps, uint16_t *q16, uint16_t *kc,
                                                                 uint16_t *vc, int max_ctx, const float *part,
                                                                 int nsplit, int ntm) {
    const int t = blockIdx.x, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int pos = pos0 + t;
    const uint16_t *row = qkv + (size_t)t * ldqkv;
    const size_t sstride = (size_t)ntm * (ldqkv / kSplitBN) * (kSplitBM * kSplitBN);
    auto elem = [&](int col) -> uint16_t {  // element (t, col) of the f16 projection
        if constexpr (SPLIT) {
            const int tl = t / kSplitBM + ntm * (col / kSplitBN);
            const float *pp = part + (size_t)tl * (kSplitBM * kSplitBN) + (t % kSplitBM) * kSplitBN + (col % kSplitBN);
            float v[kQkMaxSplit];
#pragma unroll
            for (int k = 0; k < kQkMaxSplit; ++k)
                if (k < nsplit) v[k] = pp[k * sstride];
            float sm = v[0];
#pragma unroll
            for (int k = 1; k < kQkMaxSplit; ++k)
                if (k < nsplit) sm += v[k];
            return f32_to_h16(sm);
        } else {
            return row[col];
        }
    };
    const float c = rope_cos[(size_t)pos * 64 + lane], sn = rope_sin[(size_t)pos * 64 + lane];
    const float qw0 = q_norm[lane], qw1 = q_norm[lane + 64], kw0 = k_norm[lane], kw1 = k_norm[lane + 64];
    // the wave's query and key heads h = wave, wave + 4, ... in groups of kQkMaxHeadsPerWave: every load of a
    // group (a key head's value row with it) is issued before the first is used, one memory latency per group
    for (int h0 = wave; h0 < HQ + HKV; h0 += 4 * kQkMaxHeadsPerWave) {
        uint16_t raw[kQkMaxHeadsPerWave][4];
#pragma unroll
        for (int i = 0; i < kQkMaxHeadsPerWave; ++i) {
            const int h = h0 + 4 * i;
            const int hh = h < HQ + HKV ? h : 0;
            const int src = hh * kHeadDim;  // query heads, then key heads
            const int vs = (HQ + HKV + (hh >= HQ ? hh - HQ : 0)) * kHeadDim;
            raw[i][0] = elem(src + lane);
            raw[i][1] = elem(src + lane + 64);
            raw[i][2] = elem(vs + lane);
            raw[i][3] = elem(vs + lane + 64);
        }
#pragma unroll
        for (int i = 0; i < kQkMaxHeadsPerWave; ++i) {
            const int h = h0 + 4 * i;
            if (h >= HQ + HKV) break;
            const bool is_q = h < HQ;
            const float v0 = h16_to_f32(raw[i][0]), v1 = h16_to_f32(raw[i][1]);
            const float inv = 1.0f / sqrtf(wave_sum_fast(v0 * v0 + v1 * v1) / (float)kHeadDim + eps);
            const float n0 = (is_q ? qw0 : kw0) * (v0 * inv), n1 = (is_q ? qw1 : kw1) * (v1 * inv);
            const float r0 = n0 * c - n1 * sn, r1 = n1 * c + n0 * sn;
            if (is_q) {
                // queries carry the attention scale in log2 units, 1/sqrt(128) * log2(e), applied before the f16
                // rounding so the attention kernel's scores come out of the MFMA ready for exp2
                const float qs = (1.0f / sqrtf((float)kHeadDim)) * kLog2e;
                uint16_t *dst = q16 + ((size_t)t * HQ + h) * kHeadDim;
                dst[lane] = f32_to_h16(r0 * qs);
                dst[lane + 64] = f32_to_h16(r1 * qs);
            } else {
                const int hk = h - HQ;
                const size_t at = ((size_t)hk * max_ctx + pos) * kHeadDim;
                kc[at + lane] = f32_to_bf16(r0);
                kc[at + lane + 64] = f32_to_bf16(r1);
                vc[at + lane] = f32_to_bf16(h16_to_f32(raw[i][2]));
                vc[at + lane + 64] = f32_to_bf16(h16_to_f32(raw[i][3]));
            }
        }
    }
}

// ---------------------------------------------------------------------------------------------------
// Causal GQA flash attention for T queries at positions pos0..pos0+T-1 over cache positions 0..pos0+T-1
// ([P1] section 2 item 5: query head h reads KV head floor(h / G); keys j <= the query's position).
//
// Work unit = (query block, KV head, key-range half); its eight waves cover the G query heads of that KV
// head, 16 queries per wave.  The key tiles of a query block are split into two halves run by two
// workgroups, so the longest causal rows take half as long; each half writes its per-thread softmax state
// (running max, partial sum, unnormalised output) and the later of the two to arrive merges both, always
// with the first half as the left operand, so the result does not depend on which arrives first (a prompt
// whose causal range stays within kAttnSplitKeys keys runs each unit as one workgroup over all its keys).  Work
// units are ordered longest first in the first half of the grid and shortest first in the second, so two
// workgroups resident together on a compute unit carry complementary amounts of work.  Each 64-key tile of K ([key][dim]) and V (transposed to [dim][key]) is staged in LDS once for
// all waves.  Scores are computed transposed, S^T = K Q^T, so each lane holds four keys of one query
// (query = lane%16): the row max/sum need only two cross-lane steps, and the probabilities already sit in
// the B-operand layout of O^T = V^T P^T (the k index of both operands runs over the same key set), so no
// transpose of P is needed.  Online softmax in log2 units; Q, K, V and P enter the MFMA as f16.
// ---------------------------------------------------------------------------------------------------
struct AttnPrefillArgs {
    const uint16_t *q16;      // f16 [T][HQ][128], pre-multiplied by log2(e) / sqrt(128)
    const uint16_t *ks16, *vt16;  // f16 shadow of the layer's K ([HKV][pos][128]) and V^T ([HKV][128][pos])
    int T, pos0, HQ, HKV, max_ctx;
    uint16_t *out16;          // f16 [T][HQ*128]
    unsigned *part;           // [query block][HKV][kPfState][512] f32 bits: state of the first half to finish
    unsigned *cnt;            // [query block][HKV] arrival counters, even between launches
    int *status;              // bit 4 set if a published state never arrived (bounded wait)
    int split;                // 1: the key range of each unit is split between two workgroups (see below)
};
constexpr int kPfState = 34;              // per thread: m, l, then o[32]
constexpr unsigned kPfEmpty = 0xffffffffu;  // slot word not yet published
constexpr int kPfSpin = 1 << 20;          // polling rounds before giving up (far beyond any legitimate wait)

__device__ __forceinline__ void pf_put(unsigned *p, float v) {
    __hip_atomic_store(p, __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Takes N published words p[0], p[stride], ... and restores the empty pattern: all N loads are issued
// before the first is examined (one memory round trip, not N); a word still empty is polled on its own.
// ok turns false if a wait ran out.
template <int N>
__device__ __forceinline__ void pf_take(unsigned *p, int stride, float (&out)[N], bool &ok) {
    unsigned v[N];
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = __hip_atomic_load(p + i * stride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int i = 0; i < N; ++i) {
        for (int n = 0; v[i] == kPfEmpty && n < kPfSpin; ++n) {
            __builtin_amdgcn_s_sleep(1);
            v[i] = __hip_atomic_load(p + i * stride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        ok = ok && v[i] != kPfEmpty;
        out[i] = __uint_as_float(v[i]);
    }
#pragma unroll
    for (int i = 0; i < N; ++i) __hip_atomic_store(p + i * stride, kPfEmpty, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr int kKT = 64;                  // keys per tile
// LDS rows are 64 f16 wide with a stride of 80 (160 bytes): measured free of bank conflicts for the 16-byte
// fragment reads (16 rows x four 16-byte columns per instruction), where strides of 72 or 136 cost a 2-way
// conflict.  K is kept as two such arrays (dims 0-63, 64-127); V^T rows hold the tile's 64 keys.
constexpr int kLdsLd = 80;

template <int G>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4))) void attn_prefill_kernel(AttnPrefillArgs a) {
    constexpr int NW = 8;         // waves per workgroup
    constexpr int WPH = NW / G;   // waves per query head
    constexpr int QB = 16 * WPH;  // queries per workgroup
    // two buffers of each tile: the next tile is stored while this one is multiplied (one barrier per tile);
    // 80 KB per workgroup, two workgroups per compute unit
    __shared__ __attribute__((aligned(16))) uint16_t KsB[2][2 * kKT * kLdsLd];  // [dim / 64][key][dim % 64]
    __shared__ __attribute__((aligned(16))) uint16_t VtB[2][kHeadDim * kLdsLd]; // [dim][key position]

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int nqb = (a.T + QB - 1) / QB;
    // Work unit of this workgroup.  With a multiple of 8 KV heads, the units of a head all run on one XCD
    // (workgroup j runs on XCD j mod 8), so each XCD's L2 holds only its own heads' K/V; within an XCD the
    // units go longest first in its first half and shortest first in its second.
    int half, qb, kvh;
    {
        const int j = blockIdx.x;
        const bool by_xcd = a.HKV % 8 == 0;
        const int hpg = by_xcd ? a.HKV / 8 : a.HKV;       // heads per group of units
        const int nh = a.split ? 2 : 1;                     // workgroups per (query block, KV head)
        const int nunits = nh * nqb * hpg;                  // units per group
        const int idx = by_xcd ? j >> 3 : j;
        const int rank = idx < (nunits + 1) / 2 ? idx : nunits - 1 - (idx - (nunits + 1) / 2);  // 0 = most work
        half = a.split ? rank & 1 : 0;
        qb = nqb - 1 - (rank / nh) / hpg;
        kvh = (by_xcd ? (j & 7) : 0) + (by_xcd ? 8 : 1) * ((rank / nh) % hpg);
        // uniform by construction; keeping them in scalar registers lets the tile loads use a scalar base
        half = __builtin_amdgcn_readfirstlane(half);
        qb = __builtin_amdgcn_readfirstlane(qb);
        kvh = __builtin_amdgcn_readfirstlane(kvh);
    }
    const int t0 = qb * QB;
    const int hq = kvh * G + wave / WPH;
    const int tq = t0 + (wave % WPH) * 16 + (lane & 15);  // this lane's query (C column)
    const int qpos = a.pos0 + tq;
    const int t_last = min(a.T - 1, t0 + QB - 1);
    const int n_keys = a.pos0 + t_last + 1;
    const int hsplit = a.split ? ((n_keys + kKT - 1) / kKT + 1) / 2 * kKT : n_keys;  // first key of the second half
    const int kbeg = half ? hsplit : 0;
    const int kend = half ? n_keys : min(n_keys, hsplit);
    const int g4 = lane >> 4;
    // Tiles come from the f16 shadow: the K tile is 64 rows of 256 bytes, the V^T tile 128 rows of 128 bytes
    // (64 keys already in fragment order), both copied into LDS as 16-byte chunks without conversion.  Rows
    // past the last key are in bounds (positions padded to 64) and finite; their weights are 0.
    const int ps = kv16_stride(a.max_ctx);
    const char *kbase = (const char *)(a.ks16 + (size_t)kvh * ps * kHeadDim);
    const char *vbase = (const char *)(a.vt16 + (size_t)kvh * kHeadDim * ps);
    constexpr int KCH = kKT * kHeadDim / 8 / (64 * NW);  // 16-byte chunks per thread (K; V^T the same)
    uint4 kreg[KCH], vreg[KCH];
    auto load_tile = [&](int k0v) {
        const int k0 = __builtin_amdgcn_readfirstlane(k0v);  // uniform: scalar tile base
        const char *kt = kbase + (size_t)k0 * kHeadDim * 2;
        const char *vt = vbase + (size_t)k0 * 2;
#pragma unroll
        for (int c = 0; c < KCH; ++c) {
            const int ch = tid + 64 * NW * c;
            const u32x4_t kv = *(const u32x4_t *)(kt + (unsigned)ch * 16u);  // key ch/16, dims 8*(ch%16)..
            kreg[c] = make_uint4(kv.x, kv.y, kv.z, kv.w);
            const int dim = ch >> 3, kc8 = (ch & 7) * 8;                   // V^T row dim, keys kc8..kc8+7
            const u32x4_t vv = *(const u32x4_t *)(vt + ((unsigned)dim * (unsigned)ps + (unsigned)kc8) * 2u);
            vreg[c] = make_uint4(vv.x, vv.y, vv.z, vv.w);
        }
    };
    auto store_tile = [&](int buf) {
        uint16_t *Ks = KsB[buf], *Vt = VtB[buf];
#pragma unroll
        for (int c = 0; c < KCH; ++c) {
            const int ch = tid + 64 * NW * c, key = ch >> 4, dc = (ch & 15) * 8;
            *(uint4 *)(Ks + ((dc >> 6) * kKT + key) * kLdsLd + (dc & 63)) = kreg[c];
            const int dim = ch >> 3, kc8 = (ch & 7) * 8;
            *(uint4 *)(Vt + dim * kLdsLd + kc8) = vreg[c];
        }
    };

    // Q^T fragments (B operand of S^T): lane holds Q[tq][32*ks + 8*g4 .. +8]
    uint4 qf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
        qf[ks] = tq < a.T ? *(const uint4 *)(a.q16 + ((size_t)tq * a.HQ + hq) * kHeadDim + 32 * ks + 8 * g4)
                          : make_uint4(0, 0, 0, 0);

    f32x4_t o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, l = 0.f;
    // queries enter already multiplied by log2(e) / sqrt(128) (see qknorm_rope_append_kernel)
    const int qpos_min = a.pos0 + t0 + (wave % WPH) * 16;  // first query position of this wave

    if (kbeg < kend) {
        load_tile(kbeg);
        store_tile(0);
        if (kbeg + kKT < kend) load_tile(kbeg + kKT);  // the next tile in flight during this one
    }
    __syncthreads();
    int buf = 0;
    for (int k0 = kbeg; k0 < kend; k0 += kKT, buf ^= 1) {
        const uint16_t *Ks = KsB[buf], *Vt = VtB[buf];

        // S^T tiles: lane holds scores of keys k0 + 16*kt + 4*g4 + r for its query.  Only tiles that reach
        // past the wave's first query or past the last key need the causal / length mask.
        const bool unmasked = k0 + kKT - 1 <= qpos_min && k0 + kKT <= n_keys;
        float sc[4][4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            f32x4_t sv = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const uint4 kf =
                    *(const uint4 *)(Ks + ((ks >> 1) * kKT + 16 * kt + (lane & 15)) * kLdsLd + 32 * (ks & 1) + 8 * g4);
                sv = mfma16(kf, qf[ks], sv);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) sc[kt][r] = sv[r];
        }
        if (!unmasked) {
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int kp = k0 + 16 * kt + 4 * g4 + r;
                    if (kp > qpos || kp >= n_keys) sc[kt][r] = -INFINITY;
                }
        }
        float tm = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) tm = fmaxf(tm, sc[kt][r]);
        tm = fmaxf(tm, __shfl_xor(tm, 16, 64));
        tm = fmaxf(tm, __shfl_xor(tm, 32, 64));
        // A query of the second key half may see no unmasked key yet (its max still -inf): exponentiate
        // against 0 then, which gives zero weights instead of inf - inf.
        const float mn = fmaxf(m, tm);
        const float mref = mn == -INFINITY ? 0.f : mn;
        const float alpha = __builtin_amdgcn_exp2f(m - mref);  // hardware exp2 (results below 2^-126 flush to 0)
        m = mn;
        l *= alpha;
        if (__any(alpha != 1.0f))  // once the row maxima settle most tiles leave the output unscaled
#pragma unroll
            for (int i = 0; i < 8; ++i) o[i] *= alpha;
        // probabilities as f16 pairs: P^T fragments for the two 32-key halves of the tile
        uint32_t pw[2][4];
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                const int kt0 = 2 * kb2 + (e >> 2), r0 = e & 3;
                const float p0 = __builtin_amdgcn_exp2f(sc[kt0][r0] - mref);
                const float p1 = __builtin_amdgcn_exp2f(sc[kt0][r0 + 1] - mref);
                l += p0 + p1;
                pw[kb2][e >> 1] = pack_h16x2(p0, p1);
            }
        }
        // O^T += V^T P^T: A = V^T[16 dims][32 keys] with the key set {4*g4 + 0..3, 16 + 4*g4 + 0..3}
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
            const uint4 pb = make_uint4(pw[kb2][0], pw[kb2][1], pw[kb2][2], pw[kb2][3]);
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                const uint4 vf = *(const uint4 *)(Vt + (16 * dt + (lane & 15)) * kLdsLd + 32 * kb2 + 8 * g4);
                o[dt] = mfma16(vf, pb, o[dt]);
            }
        }
        // the next tile into the other buffer (last read before the previous barrier), the one after it in
        // flight; the barrier publishes the stores and frees this buffer
        if (k0 + kKT < kend) {
            store_tile(buf ^ 1);
            if (k0 + 2 * kKT < kend) load_tile(k0 + 2 * kKT);
        }
        __syncthreads();
    }

    // Pair the two halves.  The first to arrive publishes its state and leaves; the second takes it and
    // merges.  The state slot holds the empty pattern (all ones, a NaN the arithmetic never produces) between
    // uses, and every word is stored and loaded at device scope, so the second workgroup can tell a word
    // that has not landed yet from a published one without a cache-wide fence; the merger restores the empty
    // pattern after reading.  m is uniform over the four lanes of a query; l is this lane's partial sum.
    if (a.split) {
        const size_t unit = (size_t)qb * a.HKV + kvh;
        unsigned *slot = a.part + unit * kPfState * 512 + tid;
        unsigned &s_second = *(unsigned *)&KsB[0][0];  // the tile buffers are free after the loop's last barrier
        __syncthreads();
        if (tid == 0) s_second = atomicAdd(a.cnt + unit, 1u) & 1u;
        __syncthreads();
        if (!s_second) {
            pf_put(slot, m);
            pf_put(slot + 512, l);
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) pf_put(slot + (2 + 4 * i + r) * 512, o[i][r]);
            return;
        }
        bool ok = true;
        float w[10];
        pf_take<10>(slot, 512, w, ok);  // m, l, o[0][0..3], o[1][0..3]
        const float m0 = half ? w[0] : m, m1 = half ? m : w[0];
        const float mm = fmaxf(m0, m1);
        const float s0 = exp2f(m0 - mm), s1 = exp2f(m1 - mm);
        // operands picked first, then one expression: first half's term, then the second's
        auto comb = [&](float mine, float other) {
            const float xa = half ? other : mine, xb = half ? mine : other;
            return xa * s0 + xb * s1;
        };
        l = comb(l, w[1]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            o[0][r] = comb(o[0][r], w[2 + r]);
            o[1][r] = comb(o[1][r], w[6 + r]);
        }
#pragma unroll
        for (int i = 2; i < 8; i += 2) {
            float w8[8];
            pf_take<8>(slot + (2 + 4 * i) * 512, 512, w8, ok);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                o[i][r] = comb(o[i][r], w8[r]);
                o[i + 1][r] = comb(o[i + 1][r], w8[4 + r]);
            }
        }
        if (!ok) atomicOr(a.status, kStatusTimeout);
    }
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    // the wave's 16 query rows x 128 dims staged in its own slice of the (now free) V^T buffers, then written
    // as 16-byte chunks, four whole 256-byte rows per store instruction; the same wave writes and reads its
    // slice, so no workgroup barrier is needed
    {
        constexpr int OLD = kHeadDim + 8;  // f16 per staged row
        static_assert(NW * 16 * OLD * 2 <= (int)sizeof(VtB), "output staging fits in the V^T buffers");
        uint16_t *ow = &VtB[0][0] + wave * 16 * OLD;
        const float inv = 1.0f / l;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
            for (int r = 0; r < 4; ++r) ow[(lane & 15) * OLD + 16 * dt + 4 * g4 + r] = f32_to_h16(o[dt][r] * inv);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int row = 4 * k + (lane >> 4), c8 = (lane & 15) * 8;
            const int t = t0 + (wave % WPH) * 16 + row;
            if (t < a.T)
                *(uint4 *)(a.out16 + (size_t)t * a.HQ * kHeadDim + hq * kHeadDim + c8) = *(const uint4 *)(ow + row * OLD + c8);
        }
    }
}

// Short causal ranges (every query block within kAttnSplitKeys keys) gain nothing from splitting the key range,
// whose merge costs device-scope round trips: one workgroup per (query block, KV head) then.
constexpr int kAttnSplitKeys = 256;

hipError_t launch_attn_prefill(int G, AttnPrefillArgs a, hipStream_t st) {
    const int QB = 16 * (8 / G);
    a.split = a.pos0 + a.T > kAttnSplitKeys ? 1 : 0;
    const dim3 grid((a.split ? 2 : 1) * ((a.T + QB - 1) / QB) * a.HKV);
    switch (G) {
        case 1: hipLaunchKernelGGL(attn_prefill_kernel<1>, grid, dim3(512), 0, st, a); break;
        case 2: hipLaunchKernelGGL(attn_prefill_kernel<2>, grid, dim3(512), 0, st, a); break;
        case 4: hipLaunchKernelGGL(attn_prefill_kernel<4>, grid, dim3(512), 0, st, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

int attn_prefill_qb(int G) { return G == 1 || G == 2 || G == 4 ? 16 * (8 / G) : 0; }

inline int32_t dev_rc(hipError_t e) { return e == hipSuccess ? QW3_OK : QW3_DEVICE_ERROR; }
#define QW3_PF_TRY(expr)                                  \
    do {                                                  \
        if ((expr) != hipSuccess) return QW3_DEVICE_ERROR; \
    } while (0)

}  // namespace

uint64_t attn_prefill_counter_bytes(const Dims &d) {
    const int qb = attn_prefill_qb(d.G);
    if (!d.mfma_prefill || !qb) return 0;
    return (uint64_t)((d.max_prefill + qb - 1) / qb) * d.HKV * sizeof(unsigned);
}
uint64_t attn_prefill_kv16_bytes(const Dims &d) {
    return d.mfma_prefill ? 2ull * d.HKV * kv16_stride(d.max_ctx) * kHeadDim * sizeof(uint16_t) : 0;
}
uint64_t splitk_scratch_bytes(const Dims &d) { return d.mfma_prefill ? kSplitScratchFloats * sizeof(float) : 0; }

uint64_t attn_prefill_partial_bytes(const Dims &d) {
    return attn_prefill_counter_bytes(d) / sizeof(unsigned) * kPfState * 512 * sizeof(unsigned);
}

hipError_t launch_bf16_to_f16(const void *in, void *out, size_t n, hipStream_t st) {
    hipLaunchKernelGGL(bf16_to_f16_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, (const uint16_t *)in,
                       (uint16_t *)out, n);
    return hipGetLastError();
}

// Layer stack of the tiled prefill ([P4] "Prefill versus decode": project Q/K/V for the tile, RoPE and
// publish K/V, causal attention, output and FFN projections).
int32_t prefill_layers(uint8_t *arena, const Layout &L, const Dims &d, int seq, int pos0, int T, hipStream_t st) {
    if (!d.mfma_prefill || T < 1 || T > d.max_prefill || pos0 + T > d.max_ctx) return QW3_INVALID_ARGUMENT;
    float *x = (float *)(arena + L.x);
    uint16_t *xn16 = (uint16_t *)(arena + L.xn16);
    uint16_t *qkv16 = (uint16_t *)(arena + L.qkv);  // f16 Q/K/V projections of the prefill (the f32 buffer's space)
    uint16_t *q16 = (uint16_t *)(arena + L.q16);
    uint16_t *attn16 = (uint16_t *)(arena + L.attn16);
    uint16_t *act16 = (uint16_t *)(arena + L.act16);
    const float *rc = (const float *)(arena + L.rope_cos), *rs = (const float *)(arena + L.rope_sin);
    const size_t seq_stride = (size_t)d.L * d.HKV * d.max_ctx * kHeadDim;
    uint16_t *ks16 = (uint16_t *)(arena + L.kv16);
    uint16_t *vt16 = ks16 + (size_t)d.HKV * kv16_stride(d.max_ctx) * kHeadDim;
    int *status = (int *)(arena + L.status);
    float *split_part = (float *)(arena + L.pf_split);
    // a product of a short prompt splits K when that spreads it over more workgroups
    auto product = [&](auto epi, GemmArgs g) -> hipError_t {
        constexpr int EPI = decltype(epi)::value;
        const int ns = T <= kSplitMaxT ? splitk_count(g) : 1;
        if (ns < 2) return launch_gemm<EPI>(g, st);
        g.part = split_part;
        return launch_gemm_split<EPI>(g, ns, st);
    };
    // a residual product followed by an RMSNorm (nw; null: none follows): split, the reduction also normalises;
    // returns whether xn16 now holds the normalised rows
    auto resid_product = [&](GemmArgs g, const float *nw, bool &normed) -> hipError_t {
        const int ns = T <= kSplitMaxT ? splitk_count(g) : 1;
        normed = false;
        if (ns < 2) return launch_gemm<G_RESID>(g, st);
        g.part = split_part;
        if (g.N != 1024 && g.N != 2048) return launch_gemm_split<G_RESID>(g, ns, st);  // no fused form
        normed = nw != nullptr;
        return launch_split_resid_norm(g, ns, nw, d.eps, xn16, st);
    };
    bool xn_ready = false;  // xn16 already holds this layer's normalised input
    for (int l = 0; l < d.L; ++l) {
        const uint64_t b = L.layer0 + (uint64_t)l * L.layer_stride;
        const uint16_t *wqkv = (const uint16_t *)(arena + b + L.l_wqkv16);
        const uint16_t *wo = (const uint16_t *)(arena + b + L.l_wo16);
        const uint16_t *wgu = (const uint16_t *)(arena + b + L.l_wgu16);
        const uint16_t *wd = (const uint16_t *)(arena + b + L.l_wd16);
        const size_t layer_off = (size_t)seq * seq_stride + (size_t)l * d.HKV * d.max_ctx * kHeadDim;
        uint16_t *kc = (uint16_t *)(arena + L.kcache) + layer_off;
        uint16_t *vc = (uint16_t *)(arena + L.vcache) + layer_off;

        if (!xn_ready)
            QW3_PF_TRY(launch_rmsnorm_rows(x, T, d.H, (const float *)(arena + b + L.l_attn_norm), d.eps, xn16, st));
        GemmArgs g{};
        g.A = xn16;
        g.W = wqkv;
        g.M = T;
        g.N = d.Nqkv;
        g.K = d.H;
        g.out16 = qkv16;
        g.ldo = d.Nqkv;
        // QK-Norm, RoPE and the append in the projection's epilogue (prompts past 64 tokens); with the chunk
        // starting on a 64-position boundary the epilogue also writes the chunk's part of the f16 K / V^T
        // shadow, and only the earlier positions are converted from the cache (before, so the epilogue's
        // writes land last)
        // (a short prompt whose projection splits K adds the ranges in the QK-Norm kernel instead)
        const int ns_qkv = T <= kSplitMaxT ? splitk_count(g) : 1;
        const bool fused = T > 64 && ns_qkv < 2;
        const bool fused_shadow = fused && pos0 % 64 == 0;
        if (fused_shadow && pos0 > 0)
            hipLaunchKernelGGL(kv16_convert_kernel, dim3(pos0 / 64, d.HKV, 4), dim3(256), 0, st, kc, vc, d.max_ctx, pos0,
                               ks16, vt16, status);
        if (fused) {
            g.q_norm = (const float *)(arena + b + L.l_q_norm);
            g.k_norm = (const float *)(arena + b + L.l_k_norm);
            g.rope_cos = rc;
            g.rope_sin = rs;
            g.eps = d.eps;
            g.HQ = d.HQ;
            g.HKV = d.HKV;
            g.pos0 = pos0;
            g.max_ctx = d.max_ctx;
            g.q16 = q16;
            g.kc = kc;
            g.vc = vc;
            g.ks16 = fused_shadow ? ks16 : nullptr;
            g.vt16 = fused_shadow ? vt16 : nullptr;
            g.ps = kv16_stride(d.max_ctx);
            g.status = status;
            QW3_PF_TRY(launch_gemm<G_QKNORM>(g, st));
        } else {
            // a split projection leaves its K ranges to the QK-Norm kernel, which adds them as it reads
            const int ns = ns_qkv;
            const float *qn = (const float *)(arena + b + L.l_q_norm), *kn = (const float *)(arena + b + L.l_k_norm);
            if (ns > kQkMaxSplit) {
                g.part = split_part;
                QW3_PF_TRY(launch_gemm_split<G_STORE16>(g, ns, st));
                hipLaunchKernelGGL(qknorm_rope_append_kernel<false>, dim3(T), dim3(256), 0, st, qkv16, d.Nqkv, d.HQ,
                                   d.HKV, qn, kn, rc, rs, pos0, d.eps, q16, kc, vc, d.max_ctx, nullptr, 0, 0);
            } else if (ns >= 2) {
                g.part = split_part;
                QW3_PF_TRY(launch_split_partials(g, ns, st));
                hipLaunchKernelGGL(qknorm_rope_append_kernel<true>, dim3(T), dim3(256), 0, st, qkv16, d.Nqkv, d.HQ,
                                   d.HKV, qn, kn, rc, rs, pos0, d.eps, q16, kc, vc, d.max_ctx, split_part, ns,
                                   (T + kSplitBM - 1) / kSplitBM);
            } else {
                QW3_PF_TRY(launch_gemm<G_STORE16>(g, st));
                hipLaunchKernelGGL(qknorm_rope_append_kernel<false>, dim3(T), dim3(256), 0, st, qkv16, d.Nqkv, d.HQ,
                                   d.HKV, qn, kn, rc, rs, pos0, d.eps, q16, kc, vc, d.max_ctx, nullptr, 0, 0);
            }
        }
        // every cached position of this layer (earlier chunks and the new one) into the f16 shadow
        if (!fused_shadow)
            hipLaunchKernelGGL(kv16_convert_kernel, dim3((pos0 + T + 63) / 64, d.HKV, 4), dim3(256), 0, st, kc, vc,
                               d.max_ctx, pos0 + T, ks16, vt16, status);
        AttnPrefillArgs at{};
        at.q16 = q16;
        at.ks16 = ks16;
        at.vt16 = vt16;
        at.T = T;
        at.pos0 = pos0;
        at.HQ = d.HQ;
        at.HKV = d.HKV;
        at.max_ctx = d.max_ctx;
        at.out16 = attn16;
        at.part = (unsigned *)(arena + L.pf_part);
        at.cnt = (unsigned *)(arena + L.pf_cnt);
        at.status = status;
        QW3_PF_TRY(launch_attn_prefill(d.G, at, st));
        g.A = attn16;
        g.W = wo;
        g.N = d.H;
        g.K = d.q_dim;
        g.outf = x;
        g.ldo = d.H;
        {
            bool normed;
            const float *mlp_norm = (const float *)(arena + b + L.l_mlp_norm);
            QW3_PF_TRY(resid_product(g, mlp_norm, normed));
            if (!normed) QW3_PF_TRY(launch_rmsnorm_rows(x, T, d.H, mlp_norm, d.eps, xn16, st));
        }
        g.A = xn16;
        g.W = wgu;
        g.N = 2 * d.I;
        g.K = d.H;
        g.up_off = d.I;
        g.outf = nullptr;
        g.out16 = act16;
        g.ldo = d.I;
        QW3_PF_TRY(product(std::integral_constant<int, G_SWIGLU>{}, g));
        g.A = act16;
        g.W = wd;
        g.N = d.H;
        g.K = d.I;
        g.out16 = nullptr;
        g.outf = x;
        g.ldo = d.H;
        // the next layer's attention RMSNorm rides on the down product's reduction when K is split
        const float *next_norm =
            l + 1 < d.L ? (const float *)(arena + L.layer0 + (uint64_t)(l + 1) * L.layer_stride + L.l_attn_norm) : nullptr;
        QW3_PF_TRY(resid_product(g, next_norm, xn_ready));
    }
    return dev_rc(hipGetLastError());
}

}  // namespace qw3
