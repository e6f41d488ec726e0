// Tiled bf16 prefill on MFMA (internal).
#pragma once
#include "common.h"

namespace qw3 {

// Runs every layer for T tokens of sequence `seq` whose f32 inputs are in the x scratch rows 0..T-1,
// at positions pos0..pos0+T-1, appending their K/V to the cache.  On return x holds the layer-stack output.
int32_t prefill_layers(uint8_t *arena, const Layout &L, const Dims &d, int seq, int pos0, int T, hipStream_t st);

// Sizes of the prefill attention's arrival counters and partial-state buffer for up to d.max_prefill tokens
// (zero when the tiled prefill is unavailable).  The counters live in zeroed state memory.
uint64_t attn_prefill_counter_bytes(const Dims &d);
// f16 shadow of one layer's K and V^T for the prefill attention (zeroed state memory, reused by every layer)
uint64_t attn_prefill_kv16_bytes(const Dims &d);
uint64_t attn_prefill_partial_bytes(const Dims &d);
// Prompts of up to kSplitMaxT tokens run their four products with K split over more workgroups (measured on
// 128- to 2048-token prompts: faster up to 512 tokens, no change beyond); the f32
// partial tiles take at most kSplitScratchFloats (1024 split tiles of 64 x 64, 16 MiB) in scratch memory.
constexpr int kSplitMaxT = 512;
constexpr uint64_t kSplitScratchFloats = 1024ull * 64 * 64;
uint64_t splitk_scratch_bytes(const Dims &d);

// Widens n bf16 values to f16 (round to nearest even; exact unless |v| < 2^-14 or |v| > 65504).
hipError_t launch_bf16_to_f16(const void *in, void *out, size_t n, hipStream_t st);

}  // namespace qw3
