// Host side of libqw3: handle table, shape validation, arena layout, weight upload/packing and the
// stream-ordered sequencing of the decode and prefill kernels.  See include/qw3.h for the contract.
//
// Page titles used in citations:
//   [P1] "Scalar-Native Qwen3 Reference Runtime As The Numerical Authority"
//   [P2] "M1 — Load the weights"
//   [P4] "Portable WebAssembly Runtime Architecture for TinyRustLM"
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "common.h"
#include "prefill.h"

using namespace qw3;

namespace {

// ---- checked 64-bit arithmetic ([P4] "Shape invariants": no multiplication may wrap) --------------
struct Checked {
    bool overflow = false;
    uint64_t mul(uint64_t a, uint64_t b) {
        if (a && b > UINT64_MAX / a) overflow = true;
        return a * b;
    }
    uint64_t add(uint64_t a, uint64_t b) {
        if (b > UINT64_MAX - a) overflow = true;
        return a + b;
    }
};

uint64_t align256(Checked &c, uint64_t v) { return c.add(v, 255) & ~uint64_t(255); }

struct Model {
    qw3_config_t cfg;
    Dims d;
    Layout lay;
    uint8_t *arena = nullptr;
    uint64_t arena_bytes = 0;
    std::vector<int> len;       // host mirror of the committed lengths
    bool loaded = false;
    bool poisoned = false;      // a latched device failure was observed by qw3_status_poll
    int32_t poison_code = QW3_NUMERICAL_FAILURE;  // what every call reports while poisoned
    bool lens_dirty = false;    // host lengths changed without a device update yet
    bool status_dirty = false;  // device status word must be cleared
    // Replayable decode steps: one captured graph per (tokens, logits, argmax) pointer triple.
    struct StepGraph {
        const void *tokens, *logits, *argmax;
        hipGraphExec_t exec;
    };
    std::vector<StepGraph> graphs;
    bool graphs_enabled = true;
    bool mega = false;  // single-sequence steps run as one persistent launch (decode_mega_kernel)
    bool mfma_batched = false;  // Q8 steps of 2..16 sequences run their products on MFMA (gemv_mfma.hip)
    int b1_splits = kMaxSplit / 2;  // batch-1 decode attention context splits (measured best of 16/32/64)
    ~Model() {
        for (auto &g : graphs) (void)hipGraphExecDestroy(g.exec);
    }
};

constexpr int kSlots = 64;
struct Slot {
    uint32_t generation = 0;
    Model *m = nullptr;
};
Slot g_slots[kSlots];
std::mutex g_mu;

int32_t lookup(uint64_t h, Model **out) {
    const uint32_t slot = (uint32_t)(h & 0xffffffffu), gen = (uint32_t)(h >> 32);
    if (slot >= (uint32_t)kSlots || gen == 0) return QW3_INVALID_HANDLE;
    std::lock_guard<std::mutex> lk(g_mu);
    if (g_slots[slot].generation != gen) return g_slots[slot].generation > gen ? QW3_STALE_HANDLE : QW3_INVALID_HANDLE;
    if (!g_slots[slot].m) return QW3_STALE_HANDLE;
    *out = g_slots[slot].m;
    return QW3_OK;
}

int32_t validate(const qw3_config_t *c, Dims *d) {
    if (!c) return QW3_INVALID_ARGUMENT;
    if (c->abi_version != QW3_ABI_VERSION) return QW3_UNSUPPORTED_ABI;
    if (c->weight_format != QW3_WEIGHTS_BF16 && c->weight_format != QW3_WEIGHTS_Q8 &&
        c->weight_format != QW3_WEIGHTS_Q8_0 && c->weight_format != QW3_WEIGHTS_Q8_ACT8)
        return QW3_UNSUPPORTED_QUANTIZATION;
    if (c->input_mode != QW3_INPUT_TOKENS && c->input_mode != QW3_INPUT_HIDDEN) return QW3_INVALID_ARGUMENT;
    if (c->hidden <= 0 || c->n_layers <= 0 || c->n_q_heads <= 0 || c->n_kv_heads <= 0 || c->intermediate <= 0 ||
        c->max_ctx <= 0 || c->n_seq <= 0 || c->max_prefill <= 0 || c->vocab_size < 0)
        return QW3_INVALID_ARGUMENT;
    if (!(c->rms_eps > 0.f) || !isfinite(c->rms_eps) || !(c->rope_theta > 1.0) || !isfinite(c->rope_theta))
        return QW3_INVALID_ARGUMENT;
    if (c->head_dim != kHeadDim) return QW3_UNSUPPORTED_SHAPE;
    // grouped-query attention: H_q mod H_kv = 0 ([P4] "Shape invariants")
    if (c->n_q_heads % c->n_kv_heads) return QW3_UNSUPPORTED_SHAPE;
    const int G = c->n_q_heads / c->n_kv_heads;
    if (G != 1 && G != 2 && G != 4) return QW3_UNSUPPORTED_SHAPE;
    const bool q8 = c->weight_format != QW3_WEIGHTS_BF16;  // Q8 and Q8_0 share the packed device layout
    // Q8 blocks of 32 need every contraction length to be a multiple of 32 ([P1] section 3, no tails);
    // the GEMV lane slicing needs multiples of 64 lanes x 16 bytes.
    const int unit = q8 ? 1024 : 512;
    const int q_dim = c->n_q_heads * kHeadDim;
    if (c->hidden % unit || q_dim % unit || c->intermediate % unit) return QW3_UNSUPPORTED_SHAPE;
    if (c->n_seq > kMaxSeq) return QW3_UNSUPPORTED_SHAPE;
    if (c->input_mode == QW3_INPUT_TOKENS && c->vocab_size < 1) return QW3_INVALID_ARGUMENT;
    if (c->input_mode == QW3_INPUT_HIDDEN && c->vocab_size != 0) return QW3_INVALID_ARGUMENT;
    if (c->max_ctx > (1 << 24) || c->max_prefill > (1 << 16)) return QW3_UNSUPPORTED_SHAPE;
    // the logits GEMV covers at least 16 vocabulary rows per workgroup
    if (c->input_mode == QW3_INPUT_TOKENS && c->vocab_size > kLmMaxBlocks * 16) return QW3_UNSUPPORTED_SHAPE;
    d->H = c->hidden;
    d->L = c->n_layers;
    d->HQ = c->n_q_heads;
    d->HKV = c->n_kv_heads;
    d->G = G;
    d->I = c->intermediate;
    d->V = c->vocab_size;
    d->S = c->n_seq;
    d->max_ctx = c->max_ctx;
    d->max_prefill = c->max_prefill;
    d->q_dim = q_dim;
    d->Nqkv = (c->n_q_heads + 2 * c->n_kv_heads) * kHeadDim;
    d->q8 = q8;
    d->q8_blocks = c->weight_format == QW3_WEIGHTS_Q8_0;
    d->act8 = c->weight_format == QW3_WEIGHTS_Q8_ACT8;
    d->hidden_mode = c->input_mode == QW3_INPUT_HIDDEN;
    d->mfma_prefill = !q8 && c->max_prefill > 1;
    d->eps = c->rms_eps;
    return QW3_OK;
}

// Arena layout.  Matrices keep the canonical [out, in] row-major order ([P2]); Q, K and V are stored as one
// [Nqkv, H] matrix and gate/up as one [2I, H] matrix (gate rows first) so each is streamed by one kernel.
int32_t plan(const Dims &d, Layout *lay, qw3_sizes_t *sz) {
    Checked c;
    const uint64_t eb = d.q8 ? 1 : 2;  // bytes per stored weight element
    uint64_t off = 0;
    auto take = [&](uint64_t bytes) {
        const uint64_t at = off;
        off = align256(c, c.add(off, bytes));
        return at;
    };
    auto mat = [&](uint64_t rows, uint64_t cols, uint64_t *w, uint64_t *s) {
        *w = take(c.mul(c.mul(rows, cols), eb));
        *s = d.q8 ? take(c.mul(c.mul(rows, cols / 32), 4)) : 0;
    };
    Layout L{};
    if (!d.hidden_mode) {
        mat((uint64_t)d.V, (uint64_t)d.H, &L.embed, &L.embed_scales);
        L.final_norm = take(c.mul(d.H, 4));
    }
    // one layer block, laid out relative to its start
    {
        const uint64_t save = off;
        off = 0;
        mat(d.Nqkv, d.H, &L.l_wqkv, &L.l_sqkv);
        mat(d.H, d.q_dim, &L.l_wo, &L.l_so);
        mat(c.mul(2, d.I), d.H, &L.l_wgu, &L.l_sgu);
        mat(d.H, d.I, &L.l_wd, &L.l_sd);
        L.l_attn_norm = take(c.mul(d.H, 4));
        L.l_mlp_norm = take(c.mul(d.H, 4));
        L.l_q_norm = take(kHeadDim * 4);
        L.l_k_norm = take(kHeadDim * 4);
        if (d.mfma_prefill) {
            L.l_wqkv16 = take(c.mul(c.mul(d.Nqkv, d.H), 2));
            L.l_wo16 = take(c.mul(c.mul(d.H, d.q_dim), 2));
            L.l_wgu16 = take(c.mul(c.mul(c.mul(2, d.I), d.H), 2));
            L.l_wd16 = take(c.mul(c.mul(d.H, d.I), 2));
        }
        L.layer_stride = off;
        off = save;
    }
    L.layer0 = take(c.mul(L.layer_stride, d.L));
    L.rope_cos = take(c.mul(c.mul(d.max_ctx, kHeadDim / 2), 4));
    L.rope_sin = take(c.mul(c.mul(d.max_ctx, kHeadDim / 2), 4));
    L.weights_end = off;
    const uint64_t kv_elems = c.mul(c.mul(c.mul(c.mul(d.S, d.L), d.HKV), d.max_ctx), kHeadDim);
    L.kcache = take(c.mul(kv_elems, 2));
    L.vcache = take(c.mul(kv_elems, 2));
    L.kv_end = off;
    L.len = take(kMaxSeq * 4);
    L.status = take(4);
    // single-launch decode: epoch word and tagged exchange words (8 bytes each), zeroed at load
    L.epoch = take(4);
    L.x_o = take(c.mul(xw_words(d.H), 8));
    L.x_d = take(c.mul(xw_words(d.H), 8));
    L.qkv_x = take(c.mul(d.Nqkv, 8));  // dense: measured faster than the spread lines for these words
    L.part_x = take(c.mul(c.mul((uint64_t)kMegaGrid * d.G, kPartStride), 8));  // one partial per workgroup
    L.attn_x = take(c.mul(xw_words(d.q_dim), 8));
    L.act_x = take(c.mul(xw_words(d.I), 8));
    L.pf_cnt = take(attn_prefill_counter_bytes(d));
    L.kv16 = take(attn_prefill_kv16_bytes(d));
    L.state_end = off;
    const uint64_t M = (uint64_t)(d.max_prefill > d.S ? d.max_prefill : d.S);
    L.x = take(c.mul(c.mul(M, d.H), 4));
    L.xn16 = take(c.mul(c.mul(M, d.H), 2));
    L.qkv = take(c.mul(c.mul(M, d.Nqkv), 4));
    L.q16 = take(c.mul(c.mul(M, d.q_dim), 2));
    L.attn = take(c.mul(c.mul(M, d.q_dim), 4));
    L.attn16 = take(c.mul(c.mul(M, d.q_dim), 2));
    L.act = take(c.mul(c.mul(M, d.I), 4));
    L.act16 = take(c.mul(c.mul(M, d.I), 2));
    L.part = take(c.mul(c.mul(c.mul(c.mul(d.S, d.HQ), kMaxSplit), kPartStride), 4));
    L.pf_part = take(attn_prefill_partial_bytes(d));
    L.pf_split = take(splitk_scratch_bytes(d));
    L.argpart = take(c.mul(c.mul(c.mul(kMaxSeq, kLmMaxBlocks), 2), 4));
    L.logits = d.hidden_mode ? take(0) : take(c.mul(c.mul(d.S, d.V), 4));
    L.tokens = take(c.mul(M, 4));
    L.ssq = take(c.mul(c.mul(kMaxSeq, (d.H + 15) / 16), 4));
    {
        const int kmax = d.H > d.q_dim ? (d.H > d.I ? d.H : d.I) : (d.q_dim > d.I ? d.q_dim : d.I);
        L.opnd_hi = take(c.mul(c.mul(kMaxSeq, kmax), 2));
        L.opnd_lo = take(c.mul(c.mul(kMaxSeq, kmax), 2));
    }
    L.scratch_end = off;
    if (c.overflow) return QW3_INTEGER_OVERFLOW;
    if (lay) *lay = L;
    if (sz) {
        sz->total = L.scratch_end;
        sz->weights = L.weights_end;
        sz->kv = L.kv_end - L.weights_end;
        sz->state = L.state_end - L.kv_end;
        sz->scratch = L.scratch_end - L.state_end;
    }
    return QW3_OK;
}

template <typename T>
T *at(Model *m, uint64_t off) {
    return reinterpret_cast<T *>(m->arena + off);
}

inline int32_t dev(hipError_t e) { return e == hipSuccess ? QW3_OK : QW3_DEVICE_ERROR; }
inline int weight_mode(const Dims &d) { return d.act8 ? 2 : (d.q8 ? 1 : 0); }
#define QW3_TRY(expr)                      \
    do {                                   \
        const int32_t _rc = (expr);        \
        if (_rc != QW3_OK) return _rc;     \
    } while (0)
#define QW3_HIP(expr) QW3_TRY(dev(expr))

// Bring the device length array / status word in line with the host after reset_kv / kv_set_len.
int32_t sync_state(Model *m, hipStream_t st) {
    if (!m->lens_dirty && !m->status_dirty) return QW3_OK;
    QW3_HIP(launch_set_lens(at<int>(m, m->lay.len), m->d.S, m->len.data(), (1 << m->d.S) - 1, at<int>(m, m->lay.status),
                            m->status_dirty ? 1 : 0, at<uint32_t>(m, m->lay.epoch), st));
    m->lens_dirty = m->status_dirty = false;
    return QW3_OK;
}

// ---- weight validation and upload ----------------------------------------------------------------------
struct Expect {
    int64_t rows, cols;
    int32_t dtype;
};

bool is_matrix_kind(int k) {
    return k == QW3_T_Q || k == QW3_T_K || k == QW3_T_V || k == QW3_T_O || k == QW3_T_GATE || k == QW3_T_UP ||
           k == QW3_T_DOWN;
}

Expect expected(const Dims &d, int kind) {
    const int32_t mdt = d.q8_blocks ? QW3_DT_Q8_0 : (d.q8 ? QW3_DT_Q8 : QW3_DT_BF16);
    const int32_t ndt = d.q8 ? QW3_DT_F32 : QW3_DT_BF16;
    switch (kind) {
        case QW3_T_EMBED:
        case QW3_T_LM_HEAD: return {d.V, d.H, mdt};
        case QW3_T_FINAL_NORM:
        case QW3_T_ATTN_NORM:
        case QW3_T_MLP_NORM: return {1, d.H, ndt};
        case QW3_T_Q_NORM:
        case QW3_T_K_NORM: return {1, kHeadDim, ndt};
        case QW3_T_Q: return {d.q_dim, d.H, mdt};
        case QW3_T_K:
        case QW3_T_V: return {d.HKV * kHeadDim, d.H, mdt};
        case QW3_T_O: return {d.H, d.q_dim, mdt};
        case QW3_T_GATE:
        case QW3_T_UP: return {d.I, d.H, mdt};
        case QW3_T_DOWN: return {d.H, d.I, mdt};
    }
    return {0, 0, 0};
}

uint64_t elem_bytes(int32_t dt) { return dt == QW3_DT_F32 ? 4 : (dt == QW3_DT_BF16 ? 2 : 1); }

// Bytes of a host tensor's data (a Q8_0 matrix: 34 bytes per 32 inputs).
uint64_t data_bytes(const qw3_tensor_t &t) {
    if (t.dtype == QW3_DT_Q8_0) return (uint64_t)t.rows * (uint64_t)(t.cols / 32) * 34;
    return (uint64_t)t.rows * (uint64_t)t.cols * elem_bytes(t.dtype);
}

// f16 bits -> f32, exact (every binary16 value is an f32 value)
float h16_to_f32_host(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

// A Q8_0 block's f16 scale must be finite (a NaN or infinite scale would only surface later as a numerical
// failure of every step reading that row).
bool q8_0_scales_finite(const qw3_tensor_t &t) {
    const uint8_t *b = (const uint8_t *)t.data;
    const uint64_t n = (uint64_t)t.rows * (uint64_t)(t.cols / 32);
    for (uint64_t i = 0; i < n; ++i)
        if (((b[i * 34 + 1] << 8) & 0x7c00) == 0x7c00) return false;
    return true;
}

// Host-side upload of a norm vector as f32 (bf16 widened exactly).
int32_t upload_norm(Model *m, const qw3_tensor_t &t, uint64_t off, hipStream_t st, std::vector<std::vector<float>> &keep) {
    keep.emplace_back((size_t)t.cols);
    std::vector<float> &v = keep.back();
    if (t.dtype == QW3_DT_F32) {
        memcpy(v.data(), t.data, sizeof(float) * (size_t)t.cols);
    } else {
        const uint16_t *b = (const uint16_t *)t.data;
        for (int64_t i = 0; i < t.cols; ++i) {
            const uint32_t u = (uint32_t)b[i] << 16;
            memcpy(&v[(size_t)i], &u, 4);
        }
    }
    return dev(hipMemcpyAsync(m->arena + off, v.data(), sizeof(float) * v.size(), hipMemcpyHostToDevice, st));
}

int32_t upload_matrix(Model *m, const qw3_tensor_t &t, uint64_t w_off, uint64_t s_off, uint64_t row0, hipStream_t st) {
    const uint64_t eb = m->d.q8 ? 1 : 2;
    if (t.dtype == QW3_DT_Q8_0) {
        // the pages' interleaved blocks -> the packed layout: codes [rows][cols] and f32 scales [rows][cols/32]
        const uint64_t nb = (uint64_t)t.cols / 32, n = (uint64_t)t.rows * nb;
        std::vector<int8_t> codes((size_t)(n * 32));
        std::vector<float> sc((size_t)n);
        const uint8_t *b = (const uint8_t *)t.data;
        for (uint64_t i = 0; i < n; ++i) {
            sc[i] = h16_to_f32_host((uint16_t)(b[i * 34] | (b[i * 34 + 1] << 8)));
            memcpy(&codes[i * 32], b + i * 34 + 2, 32);
        }
        QW3_HIP(hipMemcpyAsync(m->arena + w_off + row0 * (uint64_t)t.cols, codes.data(), codes.size(),
                               hipMemcpyHostToDevice, st));
        QW3_HIP(hipMemcpyAsync(m->arena + s_off + row0 * nb * 4, sc.data(), sc.size() * 4, hipMemcpyHostToDevice, st));
        return dev(hipStreamSynchronize(st));  // the staging vectors die on return
    }
    QW3_HIP(hipMemcpyAsync(m->arena + w_off + row0 * (uint64_t)t.cols * eb, t.data, (uint64_t)t.rows * t.cols * eb,
                           hipMemcpyHostToDevice, st));
    if (m->d.q8)
        QW3_HIP(hipMemcpyAsync(m->arena + s_off + row0 * (uint64_t)(t.cols / 32) * 4, t.scales,
                               (uint64_t)t.rows * (t.cols / 32) * 4, hipMemcpyHostToDevice, st));
    return QW3_OK;
}

}  // namespace

extern "C" {

uint32_t qw3_abi_version(void) { return QW3_ABI_VERSION; }

int32_t qw3_rope_table(double theta, int32_t head_dim, int32_t n_pos, float *cos_out, float *sin_out) {
    if (!cos_out || !sin_out || head_dim < 2 || head_dim % 2 || n_pos < 0 || !(theta > 1.0) || !isfinite(theta))
        return QW3_INVALID_ARGUMENT;
    // angle pos * theta^(-2i/d) for pair i, evaluated in double; cos and sin rounded once to f32
    const int half = head_dim / 2;
    std::vector<double> inv(half);
    for (int i = 0; i < half; ++i) inv[i] = pow(theta, -2.0 * (double)i / (double)head_dim);
    for (int p = 0; p < n_pos; ++p)
        for (int i = 0; i < half; ++i) {
            const double ang = (double)p * inv[i];
            cos_out[(size_t)p * half + i] = (float)cos(ang);
            sin_out[(size_t)p * half + i] = (float)sin(ang);
        }
    return QW3_OK;
}

int32_t qw3_preflight(const qw3_config_t *cfg, qw3_sizes_t *out) {
    Dims d;
    QW3_TRY(validate(cfg, &d));
    if (!out) return QW3_INVALID_ARGUMENT;
    return plan(d, nullptr, out);
}

int32_t qw3_create(const qw3_config_t *cfg, void *arena_dev, uint64_t arena_bytes, uint64_t *handle_out) {
    Dims d;
    QW3_TRY(validate(cfg, &d));
    if (!arena_dev || !handle_out) return QW3_INVALID_ARGUMENT;
    if ((uintptr_t)arena_dev & 255u) return QW3_ALIGNMENT;
    Layout lay;
    qw3_sizes_t sz;
    QW3_TRY(plan(d, &lay, &sz));
    if (arena_bytes < sz.total) return QW3_OUT_OF_MEMORY;
    Model *m = new Model();
    m->cfg = *cfg;
    m->d = d;
    m->lay = lay;
    m->arena = (uint8_t *)arena_dev;
    m->arena_bytes = arena_bytes;
    m->len.assign(d.S, 0);
    const char *ng = getenv("QW3_NO_GRAPH");
    m->graphs_enabled = !(ng && ng[0] == '1');
    const char *nm = getenv("QW3_NO_MEGA");  // run single-sequence steps kernel by kernel
    // the single-launch decode needs its whole grid resident at once: checked against the current device
    m->mega = mega_supported(d) && !(nm && nm[0] == '1') && mega_resident(weight_mode(d), d.G);
    {
        // every product of a batched step must take the MFMA path, since the residual epilogues hand the
        // next RMSNorm its sums of squares
        GemvArgs g{};
        g.S = d.S;
        bool ok = d.q8 && d.S >= 2;
        g.N = d.Nqkv, g.K = d.H;
        ok = ok && gemv_mfma_supported(g, EPI_STORE);
        g.N = d.H, g.K = d.q_dim;
        ok = ok && gemv_mfma_supported(g, EPI_RESID);
        g.N = d.I, g.K = d.H;
        ok = ok && gemv_mfma_supported(g, EPI_SWIGLU);
        g.N = d.H, g.K = d.I;
        ok = ok && gemv_mfma_supported(g, EPI_RESID);
        g.N = d.V, g.K = d.H;
        ok = ok && gemv_mfma_supported(g, EPI_LOGITS);
        m->mfma_batched = ok;
    }
    // q8 x q8 products: steps of one sequence (prefills, n_seq == 1) run in the single-launch decode, steps of
    // 2..16 sequences in the batched products' int8 form
    if (d.act8 && (!m->mega || (d.S >= 2 && !m->mfma_batched))) {
        delete m;
        return QW3_UNSUPPORTED_SHAPE;
    }
    const char *sp = getenv("QW3_B1_SPLITS");  // tuning override, 1..64
    if (sp && atoi(sp) >= 1 && atoi(sp) <= kMaxSplit) m->b1_splits = atoi(sp);
    std::lock_guard<std::mutex> lk(g_mu);
    for (int i = 0; i < kSlots; ++i) {
        if (!g_slots[i].m) {
            g_slots[i].generation += 1;
            g_slots[i].m = m;
            *handle_out = ((uint64_t)g_slots[i].generation << 32) | (uint64_t)i;
            return QW3_OK;
        }
    }
    delete m;
    return QW3_OUT_OF_MEMORY;
}

int32_t qw3_destroy(uint64_t h) {
    Model *m;
    QW3_TRY(lookup(h, &m));
    std::lock_guard<std::mutex> lk(g_mu);
    g_slots[h & 0xffffffffu].m = nullptr;
    delete m;
    return QW3_OK;
}

int32_t qw3_load_weights(uint64_t h, const qw3_tensor_t *t, int32_t n, void *stream) {
    Model *m;
    QW3_TRY(lookup(h, &m));
    if ((!t && n) || n < 0) return QW3_INVALID_ARGUMENT;
    const Dims &d = m->d;
    // ---- cross-check against the expected inventory before touching the device ([P2] cross_check)
    std::vector<int> seen_global(3, -1);
    std::vector<std::vector<int>> seen_layer(d.L, std::vector<int>(14, -1));
    for (int i = 0; i < n; ++i) {
        const qw3_tensor_t &x = t[i];
        if (x.kind < 0 || x.kind > QW3_T_DOWN) return QW3_INVALID_MODEL;
        const bool global = x.kind <= QW3_T_LM_HEAD;
        if (d.hidden_mode && global) return QW3_INVALID_MODEL;  // unexpected tensor
        if (global ? x.layer != -1 : (x.layer < 0 || x.layer >= d.L)) return QW3_INVALID_MODEL;
        int &slot = global ? seen_global[x.kind] : seen_layer[x.layer][x.kind];
        if (slot != -1) return QW3_INVALID_MODEL;  // duplicate
        slot = i;
        const Expect e = expected(d, x.kind);
        if (x.rows != e.rows || x.cols != e.cols || x.dtype != e.dtype || !x.data) return QW3_INVALID_MODEL;
        if (x.dtype == QW3_DT_Q8 && !x.scales) return QW3_INVALID_MODEL;
        if (x.dtype == QW3_DT_Q8_0 && (x.scales || !q8_0_scales_finite(x))) return QW3_INVALID_MODEL;
    }
    if (!d.hidden_mode && (seen_global[QW3_T_EMBED] < 0 || seen_global[QW3_T_FINAL_NORM] < 0))
        return QW3_INVALID_MODEL;
    for (int l = 0; l < d.L; ++l)
        for (int k = QW3_T_ATTN_NORM; k <= QW3_T_DOWN; ++k)
            if (seen_layer[l][k] < 0) return QW3_INVALID_MODEL;  // missing
    if (!d.hidden_mode && seen_global[QW3_T_LM_HEAD] >= 0) {
        // tied: a shipped lm_head must be a byte-identical copy of the embedding ([P2] "Tied != absent")
        const qw3_tensor_t &e = t[seen_global[QW3_T_EMBED]], &lm = t[seen_global[QW3_T_LM_HEAD]];
        if (memcmp(e.data, lm.data, data_bytes(e))) return QW3_INVALID_MODEL;
        if (e.dtype == QW3_DT_Q8 && memcmp(e.scales, lm.scales, (uint64_t)e.rows * (e.cols / 32) * 4))
            return QW3_INVALID_MODEL;
    }
    // ---- upload
    hipStream_t st = (hipStream_t)stream;
    std::vector<std::vector<float>> keep;
    const Layout &L = m->lay;
    if (!d.hidden_mode) {
        QW3_TRY(upload_matrix(m, t[seen_global[QW3_T_EMBED]], L.embed, L.embed_scales, 0, st));
        QW3_TRY(upload_norm(m, t[seen_global[QW3_T_FINAL_NORM]], L.final_norm, st, keep));
    }
    for (int l = 0; l < d.L; ++l) {
        const uint64_t b = L.layer0 + (uint64_t)l * L.layer_stride;
        const auto &sl = seen_layer[l];
        QW3_TRY(upload_matrix(m, t[sl[QW3_T_Q]], b + L.l_wqkv, b + L.l_sqkv, 0, st));
        QW3_TRY(upload_matrix(m, t[sl[QW3_T_K]], b + L.l_wqkv, b + L.l_sqkv, d.q_dim, st));
        QW3_TRY(upload_matrix(m, t[sl[QW3_T_V]], b + L.l_wqkv, b + L.l_sqkv, d.q_dim + d.HKV * kHeadDim, st));
        QW3_TRY(upload_matrix(m, t[sl[QW3_T_O]], b + L.l_wo, b + L.l_so, 0, st));
        QW3_TRY(upload_matrix(m, t[sl[QW3_T_GATE]], b + L.l_wgu, b + L.l_sgu, 0, st));
        QW3_TRY(upload_matrix(m, t[sl[QW3_T_UP]], b + L.l_wgu, b + L.l_sgu, d.I, st));
        QW3_TRY(upload_matrix(m, t[sl[QW3_T_DOWN]], b + L.l_wd, b + L.l_sd, 0, st));
        QW3_TRY(upload_norm(m, t[sl[QW3_T_ATTN_NORM]], b + L.l_attn_norm, st, keep));
        QW3_TRY(upload_norm(m, t[sl[QW3_T_MLP_NORM]], b + L.l_mlp_norm, st, keep));
        QW3_TRY(upload_norm(m, t[sl[QW3_T_Q_NORM]], b + L.l_q_norm, st, keep));
        QW3_TRY(upload_norm(m, t[sl[QW3_T_K_NORM]], b + L.l_k_norm, st, keep));
        if (d.mfma_prefill) {
            // f16 copies for the MFMA prefill: exact for |w| >= 2^-14, smaller magnitudes keep 2^-24 steps
            QW3_HIP(launch_bf16_to_f16(m->arena + b + L.l_wqkv, m->arena + b + L.l_wqkv16, (size_t)d.Nqkv * d.H, st));
            QW3_HIP(launch_bf16_to_f16(m->arena + b + L.l_wo, m->arena + b + L.l_wo16, (size_t)d.H * d.q_dim, st));
            QW3_HIP(launch_bf16_to_f16(m->arena + b + L.l_wgu, m->arena + b + L.l_wgu16, (size_t)2 * d.I * d.H, st));
            QW3_HIP(launch_bf16_to_f16(m->arena + b + L.l_wd, m->arena + b + L.l_wd16, (size_t)d.H * d.I, st));
        }
    }
    // RoPE table ([P1] section 2 item 4; [P4] recommends packed RoPE tables over platform libm)
    {
        const size_t n = (size_t)d.max_ctx * (kHeadDim / 2);
        std::vector<float> cs(n), sn(n);
        QW3_TRY(qw3_rope_table(m->cfg.rope_theta, kHeadDim, d.max_ctx, cs.data(), sn.data()));
        QW3_HIP(hipMemcpyAsync(m->arena + L.rope_cos, cs.data(), n * 4, hipMemcpyHostToDevice, st));
        QW3_HIP(hipMemcpyAsync(m->arena + L.rope_sin, sn.data(), n * 4, hipMemcpyHostToDevice, st));
        QW3_HIP(hipStreamSynchronize(st));
    }
    QW3_HIP(hipMemsetAsync(m->arena + L.kv_end, 0, L.state_end - L.kv_end, st));
    // prefill attention's state slots start empty (all-ones words)
    QW3_HIP(hipMemsetAsync(m->arena + L.pf_part, 0xff, attn_prefill_partial_bytes(d), st));
    QW3_HIP(hipStreamSynchronize(st));
    m->len.assign(d.S, 0);
    m->lens_dirty = m->status_dirty = false;
    m->poisoned = false;
    m->loaded = true;
    return QW3_OK;
}

int32_t qw3_reset_kv(uint64_t h, int32_t seq) {
    Model *m;
    QW3_TRY(lookup(h, &m));
    if (seq < -1 || seq >= m->d.S) return QW3_INVALID_ARGUMENT;
    for (int s = 0; s < m->d.S; ++s)
        if (seq == -1 || s == seq) m->len[s] = 0;
    m->lens_dirty = true;
    m->status_dirty = true;
    m->poisoned = false;
    m->poison_code = QW3_NUMERICAL_FAILURE;
    return QW3_OK;
}

int32_t qw3_get_len(uint64_t h, int32_t seq, int32_t *len_out) {
    Model *m;
    QW3_TRY(lookup(h, &m));
    if (seq < 0 || seq >= m->d.S || !len_out) return QW3_INVALID_ARGUMENT;
    *len_out = m->len[seq];
    return QW3_OK;
}

int32_t qw3_kv_set_len(uint64_t h, int32_t seq, int32_t len, void *stream) {
    Model *m;
    QW3_TRY(lookup(h, &m));
    if (seq < 0 || seq >= m->d.S) return QW3_INVALID_ARGUMENT;
    if (len < 0 || len > m->d.max_ctx) return QW3_BOUNDS;
    if (!m->loaded) return QW3_INVALID_ARGUMENT;
    m->len[seq] = len;
    m->lens_dirty = true;
    return sync_state(m, (hipStream_t)stream);
}

int32_t qw3_status_poll(uint64_t h, void *stream) {
    Model *m;
    QW3_TRY(lookup(h, &m));
    if (!m->loaded) return QW3_OK;
    hipStream_t st = (hipStream_t)stream;
    QW3_TRY(sync_state(m, st));
    int status = 0;
    std::vector<int> lens(m->d.S);
    QW3_HIP(hipMemcpyAsync(&status, m->arena + m->lay.status, 4, hipMemcpyDeviceToHost, st));
    QW3_HIP(hipMemcpyAsync(lens.data(), m->arena + m->lay.len, sizeof(int) * lens.size(), hipMemcpyDeviceToHost, st));
    QW3_HIP(hipStreamSynchronize(st));
    if (status) {
        // The failing step and every step after it committed nothing on the device: the host mirror takes
        // the device's committed lengths, and the handle refuses further work until qw3_reset_kv.
        m->poisoned = true;
        m->len = lens;
        if (status & kStatusTimeout) m->poison_code = QW3_DEVICE_ERROR;        // a bounded device wait gave up
        else if (status & (kStatusNonFinite | kStatusF16Range)) m->poison_code = QW3_NUMERICAL_FAILURE;
        else m->poison_code = QW3_INVALID_ARGUMENT;                            // a token outside [0, vocab)
    }
    return m->poisoned ? m->poison_code : QW3_OK;
}

// ---------------------------------------------------------------------------------------------------
// Decode sequencing.  Per layer ([P1] section 5 "Transformer Layer Execution Loop"):
//   gemv(RMSNorm -> Wqkv) -> attention (QK-Norm, RoPE, append, GQA) -> gemv(Wo) + residual
//   -> gemv(RMSNorm -> W_gate/W_up, SwiGLU) -> gemv(W_down) + residual
// then the final RMSNorm + tied logits + argmax + commit ([P1] section 2 item 7).
// ---------------------------------------------------------------------------------------------------
enum DecodeKernel { DK_QKV = 1, DK_ATTN = 2, DK_O = 3, DK_GATEUP = 4, DK_DOWN = 5 };

// Launches one kernel of layer l's decode sequence for sequences seq0..seq0+S-1.
static int32_t launch_decode_kernel(Model *m, int which, int l, int seq0, int S, hipStream_t st) {
    const Dims &d = m->d;
    const Layout &L = m->lay;
    float *x = at<float>(m, L.x);
    float *qkv = at<float>(m, L.qkv);
    float *attn = at<float>(m, L.attn);
    float *act = at<float>(m, L.act);
    const uint64_t b = L.layer0 + (uint64_t)l * L.layer_stride;
    GemvArgs g{};
    g.S = S;
    g.eps = d.eps;
    uint16_t *ohi[1] = {at<uint16_t>(m, L.opnd_hi)};
    uint16_t *olo[1] = {at<uint16_t>(m, L.opnd_lo)};
    const bool mf = m->mfma_batched && S >= 2;
    if (mf) {
        // RMSNorm inputs (Q/K/V, gate/up) come from the f32 residual stream and the sums of squares the
        // residual epilogues (o_proj, down) leave; attention writes o_proj's operand, gate/up writes down's
        g.mfma = 1;
        g.a_hi = ohi[0];
        g.a_lo = olo[0];
        g.o_hi = ohi[0];
        g.o_lo = olo[0];
        g.ssq = at<float>(m, L.ssq);
        g.ssq_mode = (which == DK_O || which == DK_DOWN) ? 2 : 1;
        g.act8 = d.act8 ? 1 : 0;  // q8 x q8: int8 activations from the f32 inputs (x, attention, activations)
    }
    switch (which) {
        case DK_QKV:  // Q/K/V projections with the pre-attention RMSNorm fused in
            g.w = m->arena + b + L.l_wqkv;
            g.scales = d.q8 ? at<float>(m, b + L.l_sqkv) : nullptr;
            g.N = d.Nqkv;
            g.K = d.H;
            g.x = x;
            g.ldx = d.H;
            g.norm_w = at<float>(m, b + L.l_attn_norm);
            g.y = qkv;
            g.ldy = d.Nqkv;
            return dev(launch_gemv(d.q8, EPI_STORE, g, st));
        case DK_ATTN: {
            const long long seq_stride = (long long)d.L * d.HKV * d.max_ctx * kHeadDim;
            int n_split = (S == 1 && m->b1_splits > 0) ? m->b1_splits : kMaxSplit / S;
            if (n_split < 1) n_split = 1;
            AttnDecodeArgs a{};
            a.qkv = qkv;
            a.ldqkv = d.Nqkv;
            a.q_norm = at<float>(m, b + L.l_q_norm);
            a.k_norm = at<float>(m, b + L.l_k_norm);
            a.rope_cos = at<float>(m, L.rope_cos);
            a.rope_sin = at<float>(m, L.rope_sin);
            const size_t layer_off = (size_t)seq0 * seq_stride + (size_t)l * d.HKV * d.max_ctx * kHeadDim;
            a.kcache = at<uint16_t>(m, L.kcache) + layer_off;
            a.vcache = at<uint16_t>(m, L.vcache) + layer_off;
            a.seq_stride = seq_stride;
            a.max_ctx = d.max_ctx;
            a.HQ = d.HQ;
            a.HKV = d.HKV;
            a.S = S;
            a.n_split = n_split;
            a.len = at<int>(m, L.len) + seq0;
            a.part = at<float>(m, L.part);
            a.out = attn;
            a.ldo = d.q_dim;
            a.eps = d.eps;
            if (mf) {
                a.o_hi = ohi[0];
                a.o_lo = olo[0];
            }
            return dev(launch_attn_decode(d.G, a, st));
        }
        case DK_O:  // o_proj + residual
            g.w = m->arena + b + L.l_wo;
            g.scales = d.q8 ? at<float>(m, b + L.l_so) : nullptr;
            g.N = d.H;
            g.K = d.q_dim;
            g.x = attn;
            g.ldx = d.q_dim;
            g.y = x;
            g.ldy = d.H;
            return dev(launch_gemv(d.q8, EPI_RESID, g, st));
        case DK_GATEUP:  // RMSNorm + gate/up + SwiGLU
            g.w = m->arena + b + L.l_wgu;
            g.scales = d.q8 ? at<float>(m, b + L.l_sgu) : nullptr;
            g.N = d.I;
            g.K = d.H;
            g.x = x;
            g.ldx = d.H;
            g.norm_w = at<float>(m, b + L.l_mlp_norm);
            g.y = act;
            g.ldy = d.I;
            return dev(launch_gemv(d.q8, EPI_SWIGLU, g, st));
        case DK_DOWN:  // down + residual
            g.w = m->arena + b + L.l_wd;
            g.scales = d.q8 ? at<float>(m, b + L.l_sd) : nullptr;
            g.N = d.H;
            g.K = d.I;
            g.x = act;
            g.ldx = d.I;
            g.y = x;
            g.ldy = d.H;
            return dev(launch_gemv(d.q8, EPI_RESID, g, st));
    }
    return QW3_INVALID_ARGUMENT;
}

static int32_t run_layers_decode(Model *m, int seq0, int S, hipStream_t st) {
    if (m->mfma_batched && S >= 2)  // sums of squares of the embedding rows for the first RMSNorm
        QW3_HIP(launch_ssq_prep(at<float>(m, m->lay.x) + (size_t)seq0 * m->d.H, m->d.H, S, m->d.H,
                                at<float>(m, m->lay.ssq), st));
    for (int l = 0; l < m->d.L; ++l)
        for (int k = DK_QKV; k <= DK_DOWN; ++k) QW3_TRY(launch_decode_kernel(m, k, l, seq0, S, st));
    return QW3_OK;
}

// Layer stack for one token of sequence `seq` in one persistent launch: input = embedding row of *token
// (token mode) or hidden_in (f32 [H]); output = x_out (f32 [H]).  Needs m->mega.
static int32_t run_layers_mega(Model *m, int seq, const int *token, const float *hidden_in, float *x_out,
                               hipStream_t st) {
    const Dims &d = m->d;
    const Layout &L = m->lay;
    MegaArgs a{};
    a.layer0 = m->arena + L.layer0;
    a.layer_stride = L.layer_stride;
    a.wqkv = L.l_wqkv;
    a.sqkv = L.l_sqkv;
    a.wo = L.l_wo;
    a.so = L.l_so;
    a.wgu = L.l_wgu;
    a.sgu = L.l_sgu;
    a.wd = L.l_wd;
    a.sd = L.l_sd;
    a.attn_norm = L.l_attn_norm;
    a.mlp_norm = L.l_mlp_norm;
    a.q_norm = L.l_q_norm;
    a.k_norm = L.l_k_norm;
    a.embed = d.hidden_mode ? nullptr : m->arena + L.embed;
    a.embed_scales = d.q8 && !d.hidden_mode ? at<float>(m, L.embed_scales) : nullptr;
    a.rope_cos = at<float>(m, L.rope_cos);
    a.rope_sin = at<float>(m, L.rope_sin);
    const size_t seq_stride = (size_t)d.L * d.HKV * d.max_ctx * kHeadDim;
    a.kcache = at<uint16_t>(m, L.kcache) + (size_t)seq * seq_stride;
    a.vcache = at<uint16_t>(m, L.vcache) + (size_t)seq * seq_stride;
    a.kv_layer_stride = (long long)d.HKV * d.max_ctx * kHeadDim;
    a.max_ctx = d.max_ctx;
    a.len = at<int>(m, L.len) + seq;
    a.token = token;
    a.hidden_in = hidden_in;
    a.x_out = x_out;
    a.status = at<int>(m, L.status);
    a.epoch = at<uint32_t>(m, L.epoch);
    a.xo = at<uint64_t>(m, L.x_o);
    a.xd = at<uint64_t>(m, L.x_d);
    a.qkv = at<uint64_t>(m, L.qkv_x);
    a.part = at<uint64_t>(m, L.part_x);
    a.attn = at<uint64_t>(m, L.attn_x);
    a.act = at<uint64_t>(m, L.act_x);
    a.L = d.L;
    a.HQ = d.HQ;
    a.HKV = d.HKV;
    a.I = d.I;
    a.V = d.V;
    a.eps = d.eps;
    return dev(launch_decode_mega(weight_mode(d), d.G, a, st));
}

static int32_t run_logits(Model *m, int seq0, int S, const float *xin, float *logits, int *argmax, int commit_add,
                          hipStream_t st) {
    const Dims &d = m->d;
    const Layout &L = m->lay;
    GemvArgs g{};
    g.S = S;
    g.eps = d.eps;
    g.w = m->arena + L.embed;
    g.scales = d.q8 ? at<float>(m, L.embed_scales) : nullptr;
    g.N = d.V;
    g.K = d.H;
    g.x = xin;
    g.ldx = d.H;
    g.norm_w = at<float>(m, L.final_norm);
    g.y = logits;
    g.ldy = d.V;
    g.argpart = at<float>(m, L.argpart);
    g.len = at<int>(m, L.len) + seq0;
    g.commit_add = commit_add;
    g.argmax_out = argmax;
    g.status = at<int>(m, L.status);
    if (m->mfma_batched && S >= 2) {  // after a batched step the last down projection left the sums of squares
        g.mfma = 1;
        g.ssq = at<float>(m, L.ssq);
        g.ssq_mode = 1;
    }
    return dev(launch_gemv(d.q8, EPI_LOGITS, g, st));
}

static int32_t check_ready(Model *m) {
    if (!m->loaded) return QW3_INVALID_ARGUMENT;
    if (m->poisoned) return m->poison_code;
    return QW3_OK;
}

static int32_t enqueue_decode_step(Model *m, const int32_t *tokens_dev, float *logits_dev, int32_t *argmax_dev,
                                   hipStream_t st) {
    const Dims &d = m->d;
    const Layout &L = m->lay;
    if (m->mega && d.S == 1) {
        QW3_TRY(run_layers_mega(m, 0, tokens_dev, nullptr, at<float>(m, L.x), st));
    } else {
        QW3_HIP(launch_embed(d.q8, m->arena + L.embed, d.q8 ? at<float>(m, L.embed_scales) : nullptr, d.H, tokens_dev,
                             d.S, at<float>(m, L.x), at<int>(m, L.status), d.V, st));
        QW3_TRY(run_layers_decode(m, 0, d.S, st));
    }
    return run_logits(m, 0, d.S, at<float>(m, L.x), logits_dev ? logits_dev : at<float>(m, L.logits), argmax_dev, 1,
                      st);
}

int32_t qw3_decode_step(uint64_t h, const int32_t *tokens_dev, float *logits_dev, int32_t *argmax_dev, void *stream) {
    Model *m;
    QW3_TRY(lookup(h, &m));
    QW3_TRY(check_ready(m));
    const Dims &d = m->d;
    if (d.hidden_mode || !tokens_dev || !argmax_dev) return QW3_INVALID_ARGUMENT;
    for (int s = 0; s < d.S; ++s)
        if (m->len[s] >= d.max_ctx) return QW3_CONTEXT_EXCEEDED;
    hipStream_t st = (hipStream_t)stream;
    QW3_TRY(sync_state(m, st));
    // The step reads positions from the device length array, so one captured graph replays any step with
    // the same buffers.  The legacy null stream cannot be captured: it runs eagerly.
    hipGraphExec_t exec = nullptr;
    if (m->graphs_enabled && st != nullptr) {
        for (auto &g : m->graphs)
            if (g.tokens == tokens_dev && g.logits == logits_dev && g.argmax == argmax_dev) exec = g.exec;
        if (!exec) {
            hipGraph_t graph = nullptr;
            bool ok = hipStreamBeginCapture(st, hipStreamCaptureModeRelaxed) == hipSuccess;
            int32_t rc = ok ? enqueue_decode_step(m, tokens_dev, logits_dev, argmax_dev, st) : QW3_OK;
            if (ok) ok = hipStreamEndCapture(st, &graph) == hipSuccess && rc == QW3_OK;
            if (ok) ok = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0) == hipSuccess;
            if (graph) (void)hipGraphDestroy(graph);
            if (!ok) {
                (void)hipGetLastError();
                exec = nullptr;
                m->graphs_enabled = false;  // this stream cannot be captured: stay eager
            } else {
                if (m->graphs.size() >= 4) {
                    (void)hipGraphExecDestroy(m->graphs.front().exec);
                    m->graphs.erase(m->graphs.begin());
                }
                m->graphs.push_back({tokens_dev, logits_dev, argmax_dev, exec});
            }
        }
    }
    if (exec)
        QW3_HIP(hipGraphLaunch(exec, st));
    else
        QW3_TRY(enqueue_decode_step(m, tokens_dev, logits_dev, argmax_dev, st));
    for (int s = 0; s < d.S; ++s) m->len[s] += 1;
    return QW3_OK;
}

// Enqueues the whole prefill of n_tokens tokens of `seq`; the caller advances the host length on success.
static int32_t enqueue_prefill(Model *m, int32_t seq, const int32_t *tokens_dev, int32_t n_tokens, float *logits,
                               int32_t *argmax, hipStream_t st) {
    const Dims &d = m->d;
    const Layout &L = m->lay;
    if (d.mfma_prefill) {
        // tiled bf16 prefill on MFMA, tile by tile ([P4] "Prefill versus decode")
        for (int t0 = 0; t0 < n_tokens; t0 += d.max_prefill) {
            const int T = n_tokens - t0 < d.max_prefill ? n_tokens - t0 : d.max_prefill;
            const bool last = t0 + T == n_tokens;
            QW3_HIP(launch_embed(false, m->arena + L.embed, nullptr, d.H, tokens_dev + t0, T, at<float>(m, L.x),
                                 at<int>(m, L.status), d.V, st));
            QW3_TRY(prefill_layers(m->arena, L, d, seq, m->len[seq] + t0, T, st));
            if (last) {
                QW3_TRY(run_logits(m, seq, 1, at<float>(m, L.x) + (size_t)(T - 1) * d.H, logits, argmax, T, st));
            } else {
                QW3_HIP(launch_commit(at<int>(m, L.len) + seq, 1, T, at<int>(m, L.status), st));
            }
        }
        return QW3_OK;
    }
    // Q8 models, and bf16 models configured with single-token tiles: token by token through the decode kernels
    // (only the last position computes logits)
    for (int t = 0; t < n_tokens; ++t) {
        if (m->mega) {
            QW3_TRY(run_layers_mega(m, seq, tokens_dev + t, nullptr, at<float>(m, L.x), st));
        } else {
            QW3_HIP(launch_embed(d.q8, m->arena + L.embed, d.q8 ? at<float>(m, L.embed_scales) : nullptr, d.H,
                                 tokens_dev + t, 1, at<float>(m, L.x), at<int>(m, L.status), d.V, st));
            QW3_TRY(run_layers_decode(m, seq, 1, st));
        }
        if (t == n_tokens - 1)
            QW3_TRY(run_logits(m, seq, 1, at<float>(m, L.x), logits, argmax, 1, st));
        else
            QW3_HIP(launch_commit(at<int>(m, L.len) + seq, 1, 1, at<int>(m, L.status), st));
    }
    return QW3_OK;
}

int32_t qw3_prefill(uint64_t h, int32_t seq, const int32_t *tokens_dev, int32_t n_tokens, float *logits_dev,
                    int32_t *argmax_dev, void *stream) {
    Model *m;
    QW3_TRY(lookup(h, &m));
    QW3_TRY(check_ready(m));
    const Dims &d = m->d;
    if (d.hidden_mode || !tokens_dev || n_tokens < 1 || seq < 0 || seq >= d.S) return QW3_INVALID_ARGUMENT;
    if ((int64_t)m->len[seq] + n_tokens > d.max_ctx) return QW3_CONTEXT_EXCEEDED;
    hipStream_t st = (hipStream_t)stream;
    QW3_TRY(sync_state(m, st));
    const Layout &L = m->lay;
    int *argmax = argmax_dev ? argmax_dev : at<int>(m, L.tokens);
    float *logits = logits_dev ? logits_dev : at<float>(m, L.logits);
    const int32_t rc = enqueue_prefill(m, seq, tokens_dev, n_tokens, logits, argmax, st);
    if (rc != QW3_OK) {
        // a launch failed part way: earlier chunks may have committed on the device, so the next call first
        // puts the device lengths back to the host's (the failed prefill commits nothing)
        m->lens_dirty = true;
        return rc;
    }
    m->len[seq] += n_tokens;
    return QW3_OK;
}

// Enqueues the layer stack over n_tokens caller hidden states of sequence 0 (qw3_block_forward).
static int32_t enqueue_block_forward(Model *m, const float *hidden_in_dev, int32_t n_tokens, float *hidden_out_dev,
                                     hipStream_t st) {
    const Dims &d = m->d;
    const Layout &L = m->lay;
    float *x = at<float>(m, L.x);
    for (int t0 = 0; t0 < n_tokens; t0 += d.max_prefill) {
        const int T = n_tokens - t0 < d.max_prefill ? n_tokens - t0 : d.max_prefill;
        if (!(m->mega && (T == 1 || d.q8)))
            QW3_HIP(hipMemcpyAsync(x, hidden_in_dev + (size_t)t0 * d.H, (size_t)T * d.H * 4, hipMemcpyDeviceToDevice,
                                   st));
        if (m->mega && (T == 1 || d.q8)) {
            for (int t = 0; t < T; ++t) {
                QW3_TRY(run_layers_mega(m, 0, nullptr, hidden_in_dev + (size_t)(t0 + t) * d.H,
                                        hidden_out_dev + (size_t)(t0 + t) * d.H, st));
                QW3_HIP(launch_commit(at<int>(m, L.len), 1, 1, at<int>(m, L.status), st));
            }
        } else if (T == 1 || d.q8) {
            for (int t = 0; t < T; ++t) {
                if (t) QW3_HIP(hipMemcpyAsync(x, hidden_in_dev + (size_t)(t0 + t) * d.H, (size_t)d.H * 4,
                                              hipMemcpyDeviceToDevice, st));
                QW3_TRY(run_layers_decode(m, 0, 1, st));
                QW3_HIP(launch_commit(at<int>(m, L.len), 1, 1, at<int>(m, L.status), st));
                QW3_HIP(hipMemcpyAsync(hidden_out_dev + (size_t)(t0 + t) * d.H, x, (size_t)d.H * 4,
                                       hipMemcpyDeviceToDevice, st));
            }
        } else {
            QW3_TRY(prefill_layers(m->arena, L, d, 0, m->len[0] + t0, T, st));
            QW3_HIP(launch_commit(at<int>(m, L.len), 1, T, at<int>(m, L.status), st));
            QW3_HIP(hipMemcpyAsync(hidden_out_dev + (size_t)t0 * d.H, x, (size_t)T * d.H * 4, hipMemcpyDeviceToDevice,
                                   st));
        }
    }
    return QW3_OK;
}

int32_t qw3_block_forward(uint64_t h, const float *hidden_in_dev, int32_t n_tokens, float *hidden_out_dev,
                          void *stream) {
    Model *m;
    QW3_TRY(lookup(h, &m));
    QW3_TRY(check_ready(m));
    const Dims &d = m->d;
    if (!d.hidden_mode || !hidden_in_dev || !hidden_out_dev || n_tokens < 1) return QW3_INVALID_ARGUMENT;
    if ((int64_t)m->len[0] + n_tokens > d.max_ctx) return QW3_CONTEXT_EXCEEDED;
    hipStream_t st = (hipStream_t)stream;
    QW3_TRY(sync_state(m, st));
    const int32_t rc = enqueue_block_forward(m, hidden_in_dev, n_tokens, hidden_out_dev, st);
    if (rc != QW3_OK) {
        m->lens_dirty = true;  // as in qw3_prefill: the failed call commits nothing
        return rc;
    }
    m->len[0] += n_tokens;
    return QW3_OK;
}

int32_t qw3_kv_write(uint64_t h, int32_t seq, int32_t layer, int32_t pos0, int32_t n_pos, const uint16_t *k_dev,
                     const uint16_t *v_dev, void *stream) {
    Model *m;
    QW3_TRY(lookup(h, &m));
    const Dims &d = m->d;
    if (!m->loaded || seq < 0 || seq >= d.S || layer < 0 || layer >= d.L || pos0 < 0 || n_pos < 0 || !k_dev || !v_dev)
        return QW3_INVALID_ARGUMENT;
    if ((int64_t)pos0 + n_pos > d.max_ctx) return QW3_BOUNDS;
    if (!n_pos) return QW3_OK;
    const size_t base = (((size_t)seq * d.L + layer) * d.HKV) * d.max_ctx * kHeadDim + (size_t)pos0 * kHeadDim;
    const size_t dpitch = (size_t)d.max_ctx * kHeadDim * 2, spitch = (size_t)n_pos * kHeadDim * 2;
    hipStream_t st = (hipStream_t)stream;
    QW3_HIP(hipMemcpy2DAsync(at<uint16_t>(m, m->lay.kcache) + base, dpitch, k_dev, spitch, spitch, d.HKV,
                             hipMemcpyDeviceToDevice, st));
    QW3_HIP(hipMemcpy2DAsync(at<uint16_t>(m, m->lay.vcache) + base, dpitch, v_dev, spitch, spitch, d.HKV,
                             hipMemcpyDeviceToDevice, st));
    return QW3_OK;
}

int32_t qw3_kv_read(uint64_t h, int32_t seq, int32_t layer, int32_t pos0, int32_t n_pos, uint16_t *k_dev,
                    uint16_t *v_dev, void *stream) {
    Model *m;
    QW3_TRY(lookup(h, &m));
    const Dims &d = m->d;
    if (!m->loaded || seq < 0 || seq >= d.S || layer < 0 || layer >= d.L || pos0 < 0 || n_pos < 0 || !k_dev || !v_dev)
        return QW3_INVALID_ARGUMENT;
    if ((int64_t)pos0 + n_pos > d.max_ctx) return QW3_BOUNDS;
    if (!n_pos) return QW3_OK;
    const size_t base = (((size_t)seq * d.L + layer) * d.HKV) * d.max_ctx * kHeadDim + (size_t)pos0 * kHeadDim;
    const size_t spitch = (size_t)d.max_ctx * kHeadDim * 2, dpitch = (size_t)n_pos * kHeadDim * 2;
    hipStream_t st = (hipStream_t)stream;
    QW3_HIP(hipMemcpy2DAsync(k_dev, dpitch, at<uint16_t>(m, m->lay.kcache) + base, spitch, dpitch, d.HKV,
                             hipMemcpyDeviceToDevice, st));
    QW3_HIP(hipMemcpy2DAsync(v_dev, dpitch, at<uint16_t>(m, m->lay.vcache) + base, spitch, dpitch, d.HKV,
                             hipMemcpyDeviceToDevice, st));
    return QW3_OK;
}

int32_t qw3_dequant(uint64_t h, int32_t kind, int32_t layer, float *out_dev, void *stream) {
    Model *m;
    QW3_TRY(lookup(h, &m));
    const Dims &d = m->d;
    const Layout &L = m->lay;
    if (!m->loaded || !out_dev) return QW3_INVALID_ARGUMENT;
    uint64_t w, s;
    long long row0 = 0;
    if (kind == QW3_T_EMBED) {
        if (d.hidden_mode) return QW3_INVALID_ARGUMENT;
        w = L.embed;
        s = L.embed_scales;
    } else if (is_matrix_kind(kind)) {
        if (layer < 0 || layer >= d.L) return QW3_INVALID_ARGUMENT;
        const uint64_t b = L.layer0 + (uint64_t)layer * L.layer_stride;
        switch (kind) {
            case QW3_T_Q: w = b + L.l_wqkv; s = b + L.l_sqkv; break;
            case QW3_T_K: w = b + L.l_wqkv; s = b + L.l_sqkv; row0 = d.q_dim; break;
            case QW3_T_V: w = b + L.l_wqkv; s = b + L.l_sqkv; row0 = d.q_dim + d.HKV * kHeadDim; break;
            case QW3_T_O: w = b + L.l_wo; s = b + L.l_so; break;
            case QW3_T_GATE: w = b + L.l_wgu; s = b + L.l_sgu; break;
            case QW3_T_UP: w = b + L.l_wgu; s = b + L.l_sgu; row0 = d.I; break;
            default: w = b + L.l_wd; s = b + L.l_sd; break;
        }
    } else {
        return QW3_INVALID_ARGUMENT;
    }
    const Expect e = expected(d, kind);
    const uint64_t eb = d.q8 ? 1 : 2;
    return dev(launch_dequant(d.q8, m->arena + w + (uint64_t)row0 * e.cols * eb,
                              d.q8 ? at<float>(m, s) + (size_t)row0 * (e.cols / 32) : nullptr, e.rows, (int)e.cols,
                              out_dev, (hipStream_t)stream));
}

int32_t qw3_bench_kernel(uint64_t h, int32_t kernel, int32_t layer, int32_t reps, void *stream) {
    Model *m;
    QW3_TRY(lookup(h, &m));
    QW3_TRY(check_ready(m));
    const Dims &d = m->d;
    if (layer < 0 || layer >= d.L || reps < 1) return QW3_INVALID_ARGUMENT;
    if (kernel < DK_QKV || kernel > 7 || (kernel == 6 && d.hidden_mode)) return QW3_INVALID_ARGUMENT;
    if (kernel == 7 && !(m->mega && d.S == 1)) return QW3_INVALID_ARGUMENT;
    if (d.act8 && kernel <= DK_DOWN) return QW3_INVALID_ARGUMENT;  // those kernels keep f32 activations
    for (int s = 0; s < d.S; ++s)
        if (m->len[s] >= d.max_ctx) return QW3_CONTEXT_EXCEEDED;
    hipStream_t st = (hipStream_t)stream;
    QW3_TRY(sync_state(m, st));
    for (int r = 0; r < reps; ++r) {
        if (kernel <= DK_DOWN)
            QW3_TRY(launch_decode_kernel(m, kernel, (layer + r) % d.L, 0, d.S, st));
        else if (kernel == 7)  // whole layer stack, in place on the scratch hidden state
            QW3_TRY(run_layers_mega(m, 0, nullptr, at<float>(m, m->lay.x), at<float>(m, m->lay.x), st));
        else
            QW3_TRY(run_logits(m, 0, d.S, at<float>(m, m->lay.x), at<float>(m, m->lay.logits), at<int>(m, m->lay.tokens),
                               0, st));
    }
    return QW3_OK;
}

}  // extern "C"
