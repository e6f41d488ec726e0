/*
 * qw3.h -- C ABI of the MI355X (gfx950) Qwen3 decoder-block library, libqw3.so.
 *
 * The library evaluates the Qwen3 decoder forward pass in the order fixed by
 * "Scalar-Native Qwen3 Reference Runtime As The Numerical Authority", section 2
 * ("Decoder-Layer Mathematical Formulation", items 1-7): RMSNorm, bias-free
 * Q/K/V projections, per-head QK-Norm, RoPE, grouped-query attention over a KV
 * cache, o_proj + residual, SwiGLU MLP + residual, then a final RMSNorm and
 * tied-embedding logits, with greedy (lowest-id-on-ties) argmax.
 *
 * ABI conventions ("Portable WebAssembly Runtime Architecture for TinyRustLM",
 * "Typed host/Wasm API" and "Generational handles"):
 *   - extern "C", fixed-width integers, no C++ types, no exceptions.
 *   - A model is named by a uint64 handle: generation << 32 | slot.  Using a
 *     destroyed handle returns QW3_STALE_HANDLE; a never-issued one
 *     QW3_INVALID_HANDLE.
 *   - Every call returns an int32 status (qw3_status_t); 0 is success.
 *
 * Memory ownership: the library never allocates device memory.  The caller
 * allocates one device arena of the size qw3_preflight reports (for example a
 * torch uint8 tensor) and keeps it alive until qw3_destroy.  The library owns
 * the layout inside the arena.  All other device pointers (tokens, logits,
 * argmax, hidden states) belong to the caller.
 *
 * Streams: `stream` is a hipStream_t passed as void* (NULL = the null stream).
 * Device work is enqueued asynchronously on it; device pointers passed to a
 * call must stay valid until the stream has passed that call.  Host-side
 * checks (arguments, shapes, context length) run before anything is enqueued:
 * when they fail, nothing is launched and no state changes.  A handle is not
 * thread-safe; use one handle per stream.
 */
#ifndef QW3_H
#define QW3_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QW3_ABI_VERSION 1u

/* Status codes; numbering follows the error taxonomy of "Portable WebAssembly Runtime Architecture for
 * TinyRustLM" ("Error taxonomy"), plus QW3_DEVICE_ERROR for a failed HIP runtime call. */
typedef enum {
    QW3_OK = 0,
    QW3_INVALID_ARGUMENT = 1,
    QW3_UNSUPPORTED_ABI = 2,
    QW3_INVALID_HANDLE = 4,
    QW3_STALE_HANDLE = 5,
    QW3_BOUNDS = 6,
    QW3_ALIGNMENT = 7,
    QW3_INTEGER_OVERFLOW = 8,
    QW3_OUT_OF_MEMORY = 9,
    QW3_INVALID_MODEL = 10,
    QW3_UNSUPPORTED_QUANTIZATION = 12,
    QW3_UNSUPPORTED_SHAPE = 13,
    QW3_CONTEXT_EXCEEDED = 14,
    QW3_NUMERICAL_FAILURE = 18,
    QW3_INTERNAL_INVARIANT = 20,
    QW3_DEVICE_ERROR = 21
} qw3_status_t;

enum { QW3_WEIGHTS_BF16 = 1, QW3_WEIGHTS_Q8 = 2, QW3_WEIGHTS_Q8_0 = 3, QW3_WEIGHTS_Q8_ACT8 = 4 };
enum { QW3_INPUT_TOKENS = 0, QW3_INPUT_HIDDEN = 1 };

/* Model and session shape.  Every field is explicit; nothing is defaulted ("M1 — Load the weights",
 * Config::load: no silent defaults).  Supported shapes (else QW3_UNSUPPORTED_SHAPE):
 *   head_dim == 128; n_q_heads % n_kv_heads == 0 and n_q_heads / n_kv_heads in {1, 2, 4};
 *   hidden, n_q_heads*128 and intermediate multiples of 512 (bf16) or 1024 (Q8);
 *   1 <= n_seq <= 16; 1 <= max_prefill; max_ctx >= 1; vocab_size >= 1 in token mode.
 * weight_format QW3_WEIGHTS_Q8 stores every matrix (projections, MLP, embedding) as int8 codes in
 * [-127, 127] with one f32 scale per 32 consecutive input elements ("Scalar-Native ...", section 3
 * "Mixed-Q8 Quantization Definition", with the scale widened to f32).  QW3_WEIGHTS_Q8_0 takes the same
 * matrices in that section's own Q8_0 block layout (QW3_DT_Q8_0 tensors: per 32 inputs one 34-byte block,
 * a little-endian f16 scale then 32 int8 codes); the packer splits the blocks into codes and scales widened
 * exactly to f32, so both formats run the same kernels and dequantize to the same f32 values.
 * QW3_WEIGHTS_Q8_ACT8 takes QW3_DT_Q8 matrices like QW3_WEIGHTS_Q8 but computes every layer projection as a
 * q8 x q8 product ("Real-Browser WASM Qwen3 Execution Under Honest Memory And Isolation Limits", section 5
 * "Q8_0 Mixed-Precision Matrix Multiplication"): the projection's input is quantized to int8 per block of 32
 * (scale max|x| / 127, codes rounded to nearest with ties away from zero, clamped to [-127, 127]), the int8
 * products of a block are summed in int32 and scaled by both block scales.  Attention, norms and the tied
 * logits keep f32 (the logits of a step of several sequences take the same f16-pair operands as in the Q8
 * format).  Steps of one sequence (every prefill, and decode with n_seq == 1) run in the single-launch decode;
 * decode steps of 2..16 sequences run the batched products with one int8 MFMA per block.  qw3_create returns
 * QW3_UNSUPPORTED_SHAPE when the device cannot hold the single-launch grid or, for n_seq >= 2, the shape has
 * no batched MFMA products.  Norm weights are bf16 in the bf16 format and f32 in the Q8 formats.
 * input_mode QW3_INPUT_HIDDEN runs the layer stack on caller-supplied f32 hidden states (no embedding,
 * no final norm, no logits; vocab_size must be 0). */
typedef struct qw3_config {
    uint32_t abi_version;   /* must equal QW3_ABI_VERSION */
    uint32_t weight_format; /* QW3_WEIGHTS_BF16, QW3_WEIGHTS_Q8, QW3_WEIGHTS_Q8_0 or QW3_WEIGHTS_Q8_ACT8 */
    uint32_t input_mode;    /* QW3_INPUT_TOKENS or QW3_INPUT_HIDDEN */
    int32_t vocab_size;
    int32_t hidden;
    int32_t n_layers;
    int32_t n_q_heads;
    int32_t n_kv_heads;
    int32_t head_dim;
    int32_t intermediate;
    int32_t max_ctx;     /* admitted context per sequence (KV positions) */
    int32_t n_seq;       /* independent sequences decoded together */
    int32_t max_prefill; /* tokens per prefill tile (longer prefills run tile by tile) */
    float rms_eps;
    double rope_theta;
} qw3_config_t;

/* Arena budget in bytes, per region; total is what qw3_create needs. */
typedef struct qw3_sizes {
    uint64_t total;
    uint64_t weights;
    uint64_t kv;
    uint64_t scratch;
    uint64_t state;
} qw3_sizes_t;

/* Tensor kinds: the per-model inventory of "M1 — Load the weights" ("What it prints", tensor table). */
enum {
    QW3_T_EMBED = 0,      /* [vocab, hidden] model.embed_tokens */
    QW3_T_FINAL_NORM = 1, /* [hidden] model.norm */
    QW3_T_LM_HEAD = 2,    /* [vocab, hidden] optional; tied: must be byte-identical to QW3_T_EMBED */
    QW3_T_ATTN_NORM = 3,  /* [hidden] input_layernorm */
    QW3_T_Q = 4,          /* [n_q_heads*head_dim, hidden] */
    QW3_T_K = 5,          /* [n_kv_heads*head_dim, hidden] */
    QW3_T_V = 6,          /* [n_kv_heads*head_dim, hidden] */
    QW3_T_Q_NORM = 7,     /* [head_dim] */
    QW3_T_K_NORM = 8,     /* [head_dim] */
    QW3_T_O = 9,          /* [hidden, n_q_heads*head_dim] */
    QW3_T_MLP_NORM = 10,  /* [hidden] post_attention_layernorm */
    QW3_T_GATE = 11,      /* [intermediate, hidden] */
    QW3_T_UP = 12,        /* [intermediate, hidden] */
    QW3_T_DOWN = 13       /* [hidden, intermediate] */
};
enum { QW3_DT_BF16 = 1, QW3_DT_F32 = 2, QW3_DT_Q8 = 3, QW3_DT_Q8_0 = 4 };

/* One canonical host tensor.  Matrices are [rows = out, cols = in] row-major (y = x W^T).
 * QW3_DT_BF16: data = uint16 bf16 bit patterns.  QW3_DT_F32: data = float.
 * QW3_DT_Q8: data = int8 codes [rows, cols], scales = float [rows, cols/32].
 * QW3_DT_Q8_0: data = uint8 blocks [rows, cols/32, 34] (bytes 0-1 the f16 scale, little-endian; bytes 2-33
 * the int8 codes of inputs 32b..32b+31), scales = NULL ("Scalar-Native ...", section 3 "The Q8_0 Block
 * Contract"; a non-finite scale is rejected with QW3_INVALID_MODEL).
 * Norm tensors are vectors: rows = 1, cols = length.  layer = -1 for global tensors. */
typedef struct qw3_tensor {
    int32_t kind;
    int32_t layer;
    int32_t dtype;
    int32_t reserved;
    int64_t rows;
    int64_t cols;
    const void *data;
    const float *scales;
} qw3_tensor_t;

/* ABI version the library was built with; a caller compares it with QW3_ABI_VERSION before any other call
 * ("Portable WebAssembly Runtime Architecture for TinyRustLM", "Typed host/Wasm API": the boundary is
 * versioned and a mismatch is a typed error, QW3_UNSUPPORTED_ABI from qw3_preflight/qw3_create). */
uint32_t qw3_abi_version(void);

/* Host-only: the RoPE cos/sin table the library uploads at load time ("Scalar-Native ...", section 2 item
 * 4, rotation of pair i by pos * theta^(-2i/head_dim); "Portable WebAssembly ..." recommends packed RoPE
 * tables over platform libm).  Angles, cos and sin are evaluated in double and rounded once to f32.
 * cos_out, sin_out: caller-owned host arrays [n_pos][head_dim/2].  Errors: QW3_INVALID_ARGUMENT for NULL
 * outputs, odd or < 2 head_dim, negative n_pos or theta <= 1.  Touches no device. */
int32_t qw3_rope_table(double theta, int32_t head_dim, int32_t n_pos, float *cos_out, float *sin_out);

/* Validates cfg and reports the arena budget.  Allocates nothing ("Portable WebAssembly Runtime ...",
 * memory formulas: preflight rejects a model/context pair before allocating).  Sizes use checked 64-bit
 * arithmetic (QW3_INTEGER_OVERFLOW on wrap).  Errors: QW3_INVALID_ARGUMENT (NULL), QW3_UNSUPPORTED_ABI,
 * QW3_UNSUPPORTED_SHAPE, QW3_UNSUPPORTED_QUANTIZATION (unknown format). */
int32_t qw3_preflight(const qw3_config_t *cfg, qw3_sizes_t *out);

/* Creates a model in a caller-owned device arena of at least qw3_preflight(cfg).total bytes, 256-byte
 * aligned (QW3_ALIGNMENT otherwise; QW3_OUT_OF_MEMORY if too small or the 64-entry handle table is full).
 * No device work is done here; the arena is initialised by qw3_load_weights.  Writes the new handle
 * (generation << 32 | slot, "Portable WebAssembly ...", "Generational handles") to *handle_out.  The
 * single-launch batch-1 decode is selected only when the current device can hold its whole grid at once
 * (occupancy query); otherwise single-sequence steps run kernel by kernel. */
int32_t qw3_create(const qw3_config_t *cfg, void *arena_dev, uint64_t arena_bytes, uint64_t *handle_out);

/* Validates and uploads the whole tensor set, packing it into the arena's device layout, then resets
 * every sequence's KV length to 0.  `tensors` lists n host tensors; each expected tensor must appear
 * exactly once with the configured shape and dtype, lm_head may be absent or byte-identical to the
 * embedding ("M1 — Load the weights", cross-check: missing, mis-shaped and unexpected tensors are
 * problems; tied lm_head may be omitted or shipped as a copy).  Any violation returns
 * QW3_INVALID_MODEL before any device work.  Host buffers are read during the call only; the call
 * returns after the copies have completed on `stream`. */
int32_t qw3_load_weights(uint64_t handle, const qw3_tensor_t *tensors, int32_t n, void *stream);

/* ---- weight files ("Scalar-Native ...", section 3 "File Layout and Safe Metadata Parsing"; "M1 — Load the
 *      weights", "The safetensors format -- three regions" and "The cross-check") -------------------------- */

/* What qw3_inspect_file found in a weight file ("M1 — Load the weights", "What it prints": tensor count and
 * the stored / logical / embedding parameter totals, a tied lm_head copy counted once in logical_params). */
typedef struct qw3_file_report {
    int64_t n_tensors;
    int64_t stored_params;
    int64_t logical_params;
    int64_t embed_params;
    int64_t header_bytes;
    int32_t n_layers;        /* highest layer index named + 1 */
    int32_t lm_head_present; /* the file ships lm_head.weight */
} qw3_file_report_t;

/* Host-only: maps `path` read-only and validates it as a safetensors container (an 8-byte little-endian
 * header length, a JSON header of {name: {dtype, shape, data_offsets}} and an optional "__metadata__" map of
 * strings, then the data blob).  Checks, in this precedence per entry: a header length beyond the file
 * (QW3_BOUNDS), malformed JSON, an unknown or duplicate name (the Qwen3 inventory: model.embed_tokens.weight,
 * model.norm.weight, optional lm_head.weight, model.layers.<l>.{input_layernorm, self_attn.{q,k,v,o}_proj,
 * self_attn.{q,k}_norm, post_attention_layernorm, mlp.{gate,up,down}_proj}.weight) or an unknown dtype
 * (BF16, F32, or Q8_0: shape [rows, cols] stored as the Q8_0 34-byte blocks of QW3_DT_Q8_0) ->
 * QW3_INVALID_MODEL; a size that does not match the shape -> QW3_INVALID_MODEL (wrapping arithmetic ->
 * QW3_INTEGER_OVERFLOW); an end offset beyond the blob -> QW3_BOUNDS; a tensor whose file offset is not a
 * multiple of 8 -> QW3_ALIGNMENT; spans that overlap, leave a hole or leave trailing bytes ->
 * QW3_INVALID_MODEL.  An unreadable path is QW3_INVALID_ARGUMENT.  Fills *out on success. */
int32_t qw3_inspect_file(const char *path, qw3_file_report_t *out);

/* Validates `path` as qw3_inspect_file does, then hands its tensors (pointing into the read-only mapping,
 * no copy on the host) to qw3_load_weights, which checks them against the handle's configuration (dtypes:
 * BF16 matrices and norms for QW3_WEIGHTS_BF16; Q8_0 matrices and F32 norms -- the SLM2 layout -- for
 * QW3_WEIGHTS_Q8_0) and uploads them.  The mapping is released before the call returns. */
int32_t qw3_load_file(uint64_t handle, const char *path, void *stream);

/* Prefill of sequence `seq`: appends n_tokens tokens at positions len..len+n_tokens-1 (KV cache, "Scalar-
 * Native ...", section 6 "Continuation and Append") and writes the last position's logits (vocab f32,
 * may be NULL) and greedy argmax (one int32, may be NULL).  tokens_dev: int32 device array [n_tokens],
 * each in [0, vocab).  len+n_tokens > max_ctx returns QW3_CONTEXT_EXCEEDED before any launch
 * (section 6 "Maximum Context Overflow": no ring buffering).  bf16 models run the tiled MFMA prefill;
 * Q8 models run token by token.  The length advances (commit) only when the step completes. */
int32_t qw3_prefill(uint64_t handle, int32_t seq, const int32_t *tokens_dev, int32_t n_tokens, float *logits_dev,
                    int32_t *argmax_dev, void *stream);

/* One greedy decode step for all n_seq sequences: tokens_dev int32 [n_seq] (may alias the previous
 * step's argmax_dev), logits_dev f32 [n_seq, vocab] (may be NULL), argmax_dev int32 [n_seq] (required).
 * Each sequence appends one position and commits len += 1.  Any sequence at len == max_ctx returns
 * QW3_CONTEXT_EXCEEDED with nothing launched.
 * Failures found on the device ("Scalar-Native ...", section 4 "NaN/Inf Rejection": a NaN or infinite
 * logit; also a token outside [0, vocab), or a cross-workgroup wait that gave up) are latched in a device
 * status word.  The failing step commits nothing, and neither does any step enqueued after it: the
 * committed lengths stay where the last good step left them (section 8: the argmax of completed steps
 * stays valid).  Calls are asynchronous, so the host learns of a latched failure only through
 * qw3_status_poll; from that poll on, every call that would launch work returns the latched code with
 * nothing launched, until qw3_reset_kv.  Logits and argmax written by the failing step and by any step
 * after it are unspecified. */
int32_t qw3_decode_step(uint64_t handle, const int32_t *tokens_dev, float *logits_dev, int32_t *argmax_dev,
                        void *stream);

/* Resets the KV length of `seq` (or of all sequences when seq == -1) to 0 and clears a latched
 * numerical failure.  No memset: old positions become unreachable because attention is bounded by the
 * length ("Scalar-Native ...", section 6 "Cancellation and Reset").  Host-side only. */
int32_t qw3_reset_kv(uint64_t handle, int32_t seq);

/* Waits for `stream` and returns the latched device status ("Scalar-Native ...", section 8: failures are
 * typed and never repaired; "Portable WebAssembly ...", "Error taxonomy"), by precedence:
 * QW3_DEVICE_ERROR when a bounded wait between workgroups gave up (the single-launch decode's workgroups
 * could not all be resident at once, e.g. because other work held the compute units), else
 * QW3_NUMERICAL_FAILURE for a non-finite logit or a cached key/value beyond the f16 range of the prefill
 * attention, else QW3_INVALID_ARGUMENT for a token id outside [0, vocab); QW3_OK when nothing is latched.
 * Any failure poisons the handle until qw3_reset_kv and sets the host's lengths (qw3_get_len) to the
 * device's committed lengths. */
int32_t qw3_status_poll(uint64_t handle, void *stream);

/* Host copy of a sequence's KV length: the length after every call enqueued so far, or, after
 * qw3_status_poll has reported a failure, the committed length the device kept ("Scalar-Native ...",
 * section 6: current_seq_len). */
int32_t qw3_get_len(uint64_t handle, int32_t seq, int32_t *len_out);

/* Releases the handle (the arena stays owned by the caller).  Later use returns QW3_STALE_HANDLE
 * ("Portable WebAssembly ...", "Generational handles": a stale handle is detected, never reused). */
int32_t qw3_destroy(uint64_t handle);

/* ---- deterministic sampling ("Scalar-Native ...", section 7 "Deterministic Sampling Contract";
 *      "Portable WebAssembly ...", "Deterministic sampling contract" and "Sampling order") ------------ */

#define QW3_SAMPLE_MAX_TOP_K 1024u   /* candidates kept by top-k when temperature > 0 */
#define QW3_SAMPLE_MAX_VOCAB 262144u
#define QW3_SAMPLE_MAX_ROWS 16u
#define QW3_SAMPLE_MAX_STOP 8u

typedef struct qw3_sample_params {
    float temperature;        /* 0: greedy (greatest logit, lowest id on ties, no draw); else positive, finite */
    float top_p;              /* (0, 1]: keep the shortest (probability desc, id asc) prefix reaching top_p */
    float repetition_penalty; /* positive, finite; 1 changes nothing */
    int32_t top_k;            /* 1..QW3_SAMPLE_MAX_TOP_K (ignored when temperature == 0) */
} qw3_sample_params_t;

/* Host-only: PCG32 state for (seed, stream_id) as "Portable WebAssembly ..." freezes its seeding (state 0,
 * increment 2*stream_id+1, advance, add the seed, advance).  state_out[0] = state, state_out[1] = increment:
 * the per-row generator layout qw3_sample reads and advances. */
int32_t qw3_pcg32_seed(uint64_t seed, uint64_t stream_id, uint64_t *state_out);

/* Bytes of device workspace qw3_sample needs for n_rows rows (QW3_INVALID_ARGUMENT outside
 * 1..QW3_SAMPLE_MAX_ROWS). */
int32_t qw3_sample_workspace_bytes(int32_t n_rows, uint64_t *bytes_out);

/* One token per row of logits, in the order of "Portable WebAssembly ...", "Sampling order" (with
 * "Scalar-Native ...", section 7): forbidden tokens -> -inf; repetition penalty on every token present in the
 * row's history (positive logits divided by the penalty, negative ones multiplied, each token once); NaN ->
 * -inf; -0 -> +0; temperature 0 -> greedy; otherwise divide by the temperature, top-k by (value desc, id asc),
 * stable probabilities over the survivors, order by (probability desc, id asc), top-p (shortest prefix whose
 * cumulative probability is at least top_p), re-normalise, and draw u = (word >> 8) * 2^-24 from the row's
 * PCG32 generator: the first candidate whose cumulative probability exceeds u.
 *   logits_dev   f32 [n_rows][ld_logits] device (ld_logits >= vocab), e.g. qw3_decode_step's logits
 *   history_dev  int32 [n_rows][n_history] device (entries outside [0, vocab) are ignored; NULL iff 0)
 *   forbid_dev   int32 [n_forbid] device, shared by all rows (NULL iff n_forbid == 0)
 *   stop_ids     host int32 [n_stop], n_stop <= QW3_SAMPLE_MAX_STOP: done_out_dev[r] = 1 when row r's token is
 *                one of them (e.g. the end-of-turn token)
 *   rng_dev      uint64 [n_rows][2] device (state, increment; see qw3_pcg32_seed); advanced by one word per row
 *                when temperature > 0, untouched at temperature 0
 *   token_out_dev int32 [n_rows] device; done_out_dev, status_out_dev int32 [n_rows] device or NULL.  A row
 *                whose logits hold +inf (or overflow when divided by the temperature) or no finite value gets
 *                token -1 and status QW3_NUMERICAL_FAILURE ("Scalar-Native ...", section 4), else QW3_OK.
 *   workspace_dev device memory of at least qw3_sample_workspace_bytes(n_rows), 256-byte aligned, owned by
 *                the caller; its contents need no initialisation.
 * Host-checked errors (nothing launched): QW3_INVALID_ARGUMENT for bad pointers, sizes or parameters
 * (penalty <= 0, temperature < 0, top_k outside 1..QW3_SAMPLE_MAX_TOP_K or top_p outside (0, 1] when
 * temperature > 0, vocab outside 1..QW3_SAMPLE_MAX_VOCAB), QW3_ALIGNMENT for a misaligned workspace,
 * QW3_OUT_OF_MEMORY for a workspace that is too small.  Asynchronous on `stream`; two launches. */
int32_t qw3_sample(const float *logits_dev, int32_t n_rows, int32_t vocab, int64_t ld_logits,
                   const qw3_sample_params_t *params, const int32_t *history_dev, int32_t n_history,
                   const int32_t *forbid_dev, int32_t n_forbid, const int32_t *stop_ids, int32_t n_stop,
                   uint64_t *rng_dev, int32_t *token_out_dev, int32_t *done_out_dev, int32_t *status_out_dev,
                   void *workspace_dev, uint64_t workspace_bytes, void *stream);

/* qw3_sample for callers that cannot allocate device memory -- code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc: the same arguments and results without the workspace.  Its scratch
 * (2,099,200 bytes, enough for QW3_SAMPLE_MAX_ROWS rows of any supported vocabulary) is a device array inside
 * the library, one per GPU, held until the process ends; the call itself allocates nothing.  Requests beyond
 * QW3_SAMPLE_MAX_ROWS rows or QW3_SAMPLE_MAX_VOCAB tokens are rejected with QW3_INVALID_ARGUMENT.  Every call
 * on a GPU uses that GPU's one array, so calls that overlap on one GPU (different streams, or host threads
 * without ordering) race and must not be issued; calls ordered on one stream are safe.  Nothing in the array
 * needs clearing between calls: each call writes every word it reads.  QW3_DEVICE_ERROR if the array's device
 * address cannot be obtained. */
int32_t qw3_sample_noalloc(const float *logits_dev, int32_t n_rows, int32_t vocab, int64_t ld_logits,
                           const qw3_sample_params_t *params, const int32_t *history_dev, int32_t n_history,
                           const int32_t *forbid_dev, int32_t n_forbid, const int32_t *stop_ids, int32_t n_stop,
                           uint64_t *rng_dev, int32_t *token_out_dev, int32_t *done_out_dev, int32_t *status_out_dev,
                           void *stream);

/* ---- test and benchmark hooks (not part of the serving path) ------------------------------------- */

/* Layer stack on caller hidden states (input_mode QW3_INPUT_HIDDEN, sequence 0): hidden_in_dev f32
 * [n_tokens, hidden] at positions len..len+n_tokens-1, writes hidden_out_dev f32 [n_tokens, hidden]
 * (every position's output).  n_tokens == 1 runs the decode kernels, n_tokens > 1 the prefill kernels. */
int32_t qw3_block_forward(uint64_t handle, const float *hidden_in_dev, int32_t n_tokens, float *hidden_out_dev,
                          void *stream);

/* Writes n_pos cache positions of one (seq, layer): k_dev, v_dev bf16 bits [n_kv_heads, n_pos, head_dim].
 * Does not change the length.  QW3_BOUNDS when pos0+n_pos > max_ctx. */
int32_t qw3_kv_write(uint64_t handle, int32_t seq, int32_t layer, int32_t pos0, int32_t n_pos, const uint16_t *k_dev,
                     const uint16_t *v_dev, void *stream);

/* Reads n_pos cache positions of one (seq, layer) into k_dev, v_dev (same layout as qw3_kv_write). */
int32_t qw3_kv_read(uint64_t handle, int32_t seq, int32_t layer, int32_t pos0, int32_t n_pos, uint16_t *k_dev,
                    uint16_t *v_dev, void *stream);

/* Sets the committed KV length of `seq` (after qw3_kv_write; "Scalar-Native ...", section 6, the session's
 * current_seq_len).  QW3_BOUNDS when len > max_ctx, QW3_INVALID_ARGUMENT for a bad seq or before
 * qw3_load_weights. */
int32_t qw3_kv_set_len(uint64_t handle, int32_t seq, int32_t len, void *stream);

/* Dequantized f32 copy of a packed matrix as the kernels read it: kind in QW3_T_Q..QW3_T_DOWN (with
 * layer) or QW3_T_EMBED; out_dev f32 [rows, cols].  For Q8 each element is one f32 multiply code*scale. */
int32_t qw3_dequant(uint64_t handle, int32_t kind, int32_t layer, float *out_dev, void *stream);

/* Launches one kernel of the decode step `reps` times back to back on the current state, for timing:
 * kernel 1 = RMSNorm+QKV GEMV, 2 = attention (re-appends the current position's K/V), 3 = o_proj+residual,
 * 4 = RMSNorm+gate/up+SwiGLU, 5 = down+residual (layers layer, layer+1, ... cyclically), 6 = final norm +
 * logits + argmax (no commit), 7 = the whole layer stack of sequence 0 as one persistent launch (only for
 * single-sequence models whose shape that kernel covers; QW3_INVALID_ARGUMENT otherwise).  Lengths do not
 * advance; the residual-updating kernels change the scratch hidden state, so a step after this hook is not a
 * continuation of the previous one. */
int32_t qw3_bench_kernel(uint64_t handle, int32_t kernel, int32_t layer, int32_t reps, void *stream);

/* Measurement probes (not part of the forward pass): attainable peaks on the current device, so that roofline
 * fractions can be stated against both the nominal peak and what a plain kernel reaches.
 * qw3_probe_hbm_read streams `bytes` (16-byte aligned device buffer) once with 16-byte nontemporal loads on
 * `grid` workgroups of 256 threads, writing one word per workgroup to out_dev (uint32 [grid]).
 * qw3_probe_mfma_f16 runs `iters` rounds of sixteen independent v_mfma_f32_16x16x32_f16 per wave on `grid`
 * workgroups of four waves (16384 flops per instruction), writing one float per wave to out_dev
 * (float [grid * 4]).  QW3_INVALID_ARGUMENT for null or misaligned pointers, grid outside 1..65536. */
int32_t qw3_probe_hbm_read(const void *buf_dev, uint64_t bytes, uint32_t *out_dev, int32_t grid, void *stream);
int32_t qw3_probe_mfma_f16(int32_t iters, int32_t grid, float *out_dev, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* QW3_H */
