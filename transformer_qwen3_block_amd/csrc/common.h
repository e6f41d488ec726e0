// Internal declarations shared by the host side and the gfx950 kernels of libqw3.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qw3.h"

namespace qw3 {

constexpr int kHeadDim = 128;
constexpr int kMaxSeq = 16;
constexpr int kMaxSplit = 64;          // decode attention splits of the context per (seq, kv head)
constexpr int kPartStride = 2 + kHeadDim;  // per split partial: running max, running sum, o[128]
constexpr int kLmMaxBlocks = 16384;    // upper bound on lm_head workgroups (argmax partials)
constexpr int kMegaGrid = 256;         // resident workgroups of the single-launch decode kernel
constexpr int kMegaWaves = 4;          // its waves per workgroup
// Bits of the device status word (zeroed at load and by qw3_reset_kv).  Any set bit stops every later commit.
constexpr int kStatusNonFinite = 1;    // a logit was NaN or infinite
constexpr int kStatusBadToken = 2;     // a token id outside [0, vocab) reached the device (row 0 was used)
constexpr int kStatusTimeout = 4;      // a bounded cross-workgroup wait gave up
constexpr int kStatusF16Range = 8;     // a cached key or value overflowed the f16 range of the prefill attention
// The single-launch decode kernel's all-gathered exchange words (hidden rows, attention output, activations)
// sit 16 to a 128-byte line, with consecutive lines kXwLine words (1 KiB) apart: measured on gfx950, packing
// those lines densely (each line written from four XCDs and polled by every workgroup) made the layer stack
// about 4 % slower.  The Q/K/V words, which each workgroup polls only for its own KV head, measured faster
// dense.
constexpr int kXwLine = 128;
__host__ __device__ inline int xw_index(int i) { return (i >> 4) * kXwLine + (i & 15); }  // 32-bit: keeps the poll addressing in 32-bit offsets
// Those words are written in kXwReps copies, one per XCD: every workgroup polls its own XCD's copy, so a line
// is polled by 32 workgroups instead of 256.  Copy r of an n-word vector starts r * xw_rep(n) words in.
constexpr int kXwReps = 8;
__host__ __device__ inline int xw_rep(int n) { return ((n + 15) / 16) * kXwLine; }
inline uint64_t xw_words(int n) { return (uint64_t)xw_rep(n) * kXwReps; }

// Byte offsets of every region inside the caller's arena.  Per-layer weight blocks repeat with a fixed
// stride, so layer l's block starts at layer0 + l * layer_stride.
struct Layout {
    // weights
    uint64_t embed, embed_scales, final_norm;
    uint64_t layer0, layer_stride;
    uint64_t l_wqkv, l_sqkv, l_wo, l_so, l_wgu, l_sgu, l_wd, l_sd;  // relative to the layer block
    uint64_t l_attn_norm, l_mlp_norm, l_q_norm, l_k_norm;           // f32 vectors
    uint64_t l_wqkv16, l_wo16, l_wgu16, l_wd16;  // f16 copies of the bf16 projections (MFMA prefill), or 0
    uint64_t rope_cos, rope_sin;                                     // f32 [max_ctx][head_dim/2]
    // KV cache, bf16 [seq][layer][kv_head][pos][head_dim]
    uint64_t kcache, vcache;
    // state
    uint64_t len, status;
    // single-launch decode: epoch tag base and the tagged exchange words (f32 value | tag << 32)
    uint64_t epoch, x_o, x_d, qkv_x, part_x, attn_x, act_x;
    // prefill attention: arrival counters of the two key-range halves of each (query block, KV head), and
    // the f16 shadow of a layer's K / V^T
    uint64_t pf_cnt, kv16;
    // scratch
    uint64_t x, xn16, qkv, q16, attn, attn16, act, act16, part, argpart, logits, tokens, ssq;
    uint64_t opnd_hi, opnd_lo;  // batched Q8 products: f16 operand pair handed from a kernel to the next product
    uint64_t pf_part;           // prefill attention: per-thread partial softmax state of each key-range half
    uint64_t pf_split;          // prefill products of short prompts: f32 partial tiles of the K ranges
    uint64_t weights_end, kv_end, state_end, scratch_end;
};

// Shape constants derived from the configuration.
struct Dims {
    int H, L, HQ, HKV, G, I, V, S, max_ctx, max_prefill;
    int Nqkv;        // (HQ + 2*HKV) * 128
    int q_dim;       // HQ * 128
    bool q8;            // int8 codes + f32 scales on the device (Q8 and Q8_0 formats)
    bool q8_blocks;     // matrices arrive as Q8_0 34-byte blocks (f16 scale), split by the packer
    bool act8;          // layer products quantize their activations to int8 per 32-block (q8 x q8)
    bool hidden_mode;
    bool mfma_prefill;  // bf16 weights and multi-token tiles: f16 weight copies exist
    float eps;
};

// ---- device helpers -------------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// f32 -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x7fffffu)) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte streaming load (read-once data: weights, KV cache).
__device__ __forceinline__ uint4 load_nt16(const void *p) {
    const u32x4_t v = __builtin_nontemporal_load((const u32x4_t *)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// DPP lane moves (VALU; no LDS round trip).  Controls: quad_perm [1,0,3,2] = 0xB1, [2,3,0,1] = 0x4E,
// row_half_mirror = 0x141, row_mirror = 0x140 (a row is 16 lanes).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
// Sum over the 16 lanes of each row, in every lane of the row.
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_mov<0xB1>(v);
    v += dpp_mov<0x4E>(v);
    v += dpp_mov<0x141>(v);
    v += dpp_mov<0x140>(v);
    return v;
}
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, dpp_mov<0xB1>(v));
    v = fmaxf(v, dpp_mov<0x4E>(v));
    v = fmaxf(v, dpp_mov<0x141>(v));
    v = fmaxf(v, dpp_mov<0x140>(v));
    return v;
}
__device__ __forceinline__ float lane_get(float v, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
// Sums over the two halves of the wave (lanes l and l + 32) and over row pairs (odd and even rows of 16
// lanes), two values per register swap: v_permlane32_swap / v_permlane16_swap exchange half of one register
// with half of another, so a + b of the swapped pair folds two values at once.
__device__ __forceinline__ float swap32_sum(float a, float b) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float swap16_sum(float a, float b) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
// Whole-wave sum / max, wave-uniform result: row reductions on DPP, then the four row results.
__device__ __forceinline__ float wave_sum_fast(float v) {
    v = row16_sum(v);
    return (lane_get(v, 0) + lane_get(v, 16)) + (lane_get(v, 32) + lane_get(v, 48));
}
__device__ __forceinline__ float wave_max_fast(float v) {
    v = row16_max(v);
    return fmaxf(fmaxf(lane_get(v, 0), lane_get(v, 16)), fmaxf(lane_get(v, 32), lane_get(v, 48)));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

// ---- launchers (stream-ordered, no host synchronisation) ------------------------------------------
enum GemvEpi { EPI_STORE = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_LOGITS = 3 };

struct GemvArgs {
    const void *w;          // bf16 bits or int8 codes, [rows][K]
    const float *scales;    // Q8: [rows][K/32]
    int N;                  // output units (rows; SwiGLU: gate/up pairs, up rows start at row N)
    int K;
    int S;                  // vectors (sequences)
    const float *x;         // input [S][ldx]
    int ldx;
    const float *norm_w;    // optional RMSNorm weight applied to x first (f32 [K])
    float eps;
    float *y;               // output [S][ldy]
    int ldy;
    // EPI_LOGITS only
    float *argpart;         // [S][gridDim.x][2]
    int *len;               // committed lengths of the S sequences (indexed from seq0)
    int commit_add;
    int *argmax_out;        // [S]
    int *status;
    // Batched Q8 path on MFMA (2..16 sequences), see gemv_mfma.hip.  Activations travel between the kernels
    // of a step as MFMA operands: f16 high part and f16 remainder, [K/64][4][kMaxSeq][16] each.
    int mfma;               // nonzero: take the MFMA path (the caller checked gemv_mfma_supported)
    const uint16_t *a_hi, *a_lo;  // operand of a product without RMSNorm (o_proj: attention, down: activations)
    uint16_t *o_hi, *o_lo;        // operand written for the next product (SwiGLU epilogue)
    float *ssq;             // [H/16][kMaxSeq] per 16-row tile sums of squares of the residual stream
    int ssq_mode;           // 1: RMSNorm input, 1/rms from ssq; 2: the residual epilogue writes ssq
    int act8;               // q8 x q8: activations quantized to int8 per block, products on int8 MFMA (not logits)
};
// Index of activation element k of sequence s in an MFMA operand buffer: [K/64][4][kMaxSeq][16], so the lane
// of column group g and sequence s reads columns 16g..16g+15 of a 64-column block pair as one 32-byte run.
__host__ __device__ inline size_t mfma_opnd_index(int k, int s) {
    return ((size_t)((k >> 6) * 4 + ((k >> 4) & 3)) * kMaxSeq + s) * 16 + (k & 15);
}

hipError_t launch_gemv(bool q8, GemvEpi epi, const GemvArgs &a, hipStream_t st);
bool gemv_mfma_supported(const GemvArgs &a, GemvEpi epi);
hipError_t launch_gemv_mfma(GemvEpi epi, const GemvArgs &a, hipStream_t st);
hipError_t launch_ssq_prep(const float *x, int ldx, int S, int K, float *ssq, hipStream_t st);
hipError_t launch_argmax_finalize(const float *argpart, int nparts, int S, int *argmax_out, int *len, int commit_add,
                                  const int *status, hipStream_t st);

struct AttnDecodeArgs {
    const float *qkv;       // raw projections [S][ldqkv]
    int ldqkv;
    const float *q_norm, *k_norm;   // f32 [128]
    const float *rope_cos, *rope_sin;
    uint16_t *kcache, *vcache;      // base of (seq0, layer) head 0: [HKV][max_ctx][128]
    long long seq_stride;           // elements between consecutive sequences' blocks of this layer
    int max_ctx, HQ, HKV, S, n_split;
    const int *len;                 // [S] (already offset to seq0)
    float *part;                    // [S][HQ][kMaxSplit][kPartStride]
    float *out;                     // [S][ldo]
    int ldo;
    float eps;
    uint16_t *o_hi, *o_lo;          // optional: the output also as MFMA operands (batched Q8 products)
};
hipError_t launch_attn_decode(int G, const AttnDecodeArgs &a, hipStream_t st);

// Single-launch decode of one token of one sequence (hidden size 1024): the whole layer stack in one
// persistent grid of kMegaGrid workgroups (see mega.hip).
struct MegaArgs {
    const uint8_t *layer0;  // first layer block; layer l at layer0 + l * layer_stride
    uint64_t layer_stride;
    uint64_t wqkv, sqkv, wo, so, wgu, sgu, wd, sd, attn_norm, mlp_norm, q_norm, k_norm;  // offsets in a block
    const void *embed;
    const float *embed_scales;
    const float *rope_cos, *rope_sin;
    uint16_t *kcache, *vcache;   // (sequence, layer 0, KV head 0)
    long long kv_layer_stride;   // elements between consecutive layers of the sequence
    int max_ctx;
    const int *len;              // committed length of the sequence (= position of the new token)
    const int *token;            // token id (token mode) or nullptr
    const float *hidden_in;      // f32 [1024] input (hidden mode) or nullptr
    float *x_out;                // f32 [1024] output of the layer stack
    int *status;
    uint32_t *epoch;             // tag base; advanced by the launch for the next one
    uint64_t *xo, *xd, *qkv, *part, *attn, *act;  // tagged exchange words
    int L, HQ, HKV, I, V;
    float eps;
};
bool mega_supported(const Dims &d);
// weight mode: 0 bf16, 1 Q8 (f32 activations), 2 Q8 with int8-quantized activations (q8 x q8)
bool mega_resident(int wmode, int G);
hipError_t launch_decode_mega(int wmode, int G, const MegaArgs &a, hipStream_t st);

// Deterministic sampling (sample.hip): vocabulary slices of the chunk kernel, bounds of the C ABI.
constexpr int kSampleChunks = 16;
constexpr int kSampleMaxTopK = QW3_SAMPLE_MAX_TOP_K;
constexpr int kSampleMaxVocab = QW3_SAMPLE_MAX_VOCAB;
constexpr int kSampleMaxRows = QW3_SAMPLE_MAX_ROWS;
constexpr int kSampleMaxStop = QW3_SAMPLE_MAX_STOP;
struct SampleArgs {
    const float *logits;    // [rows][ld]
    long long ld;
    int V, rows;
    float temperature, top_p, penalty;
    int top_k;              // 1 when temperature == 0 (greedy)
    const int *history;     // [rows][n_history]
    int n_history;
    const int *forbid;      // [n_forbid]
    int n_forbid;
    int stop[kSampleMaxStop];
    int n_stop;
    uint64_t *rng;          // [rows][2]: PCG32 state, increment
    int *token_out, *done_out, *status_out;
    // scratch (sample_bind_scratch): per (row, chunk) candidates, counts and +inf flags
    uint32_t *cand_key;
    int *cand_id, *cand_cnt, *chunk_bad;
};
uint64_t sample_scratch_bytes(int rows);
void sample_bind_scratch(SampleArgs &a, void *scratch);
hipError_t launch_sample(const SampleArgs &a, hipStream_t st);

hipError_t launch_embed(bool q8, const void *table, const float *scales, int H, const int *tokens, int S, float *x,
                        int *status, int vocab, hipStream_t st);
hipError_t launch_set_lens(int *len_dev, int n, const int *vals, int mask, int *status, int clear_status,
                           uint32_t *epoch, hipStream_t st);
hipError_t launch_commit(int *len_dev, int n, int add, const int *status, hipStream_t st);
hipError_t launch_dequant(bool q8, const void *w, const float *scales, long long rows, int cols, float *out,
                          hipStream_t st);

}  // namespace qw3
