"""Pins for the oracle: each test checks it against something other than itself.

Sources of truth used here: closed forms and invariants of the operations on
"Scalar-Native Qwen3 Reference Runtime As The Numerical Authority" (section 2
equations, section 7 softmax, section 9 hand-check vectors), the integers
printed on "M1 — Load the weights", library routines that compute the same
special case (HF transformers' Qwen3 model and rotary helper, in fp64), the
fp64 matrix-form twin, and brute force on tiny inputs.
"""
import json
import math
import os
from dataclasses import replace

import numpy as np
import pytest

import oracle
import synth
from oracle import twin64

U = 2.0 ** -24
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

TINY = replace(synth.QWEN3_06B, vocab=97, hidden=64, n_layers=2, n_q_heads=4, n_kv_heads=2, head_dim=16, inter=96,
               max_ctx=16)


def gamma(n):
    return n * U / (1 - n * U)


# ---------------------------------------------------------------------------------------------- inputs
def test_pcg32_known_answer():
    """PCG32 transition/output/seeding as defined on the 'Portable WebAssembly Runtime' page reproduce
    the published PCG32 known-answer words for seed 42, stream 54."""
    kat = json.load(open(os.path.join(GOLDEN, "pcg32_kat.json")))
    got = synth.pcg32_words(kat["seed"], kat["stream"], len(kat["words"]))
    assert [int(x, 16) for x in kat["words"]] == got.tolist()


def test_synth_deterministic():
    a = synth.normal_bf16(7, 3, (1000,))
    b = synth.normal_bf16(7, 3, (1000,))
    c = synth.normal_bf16(8, 3, (1000,))
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    codes = synth.int8_uniform(7, 4, (200000,))
    assert codes.min() == -127 and codes.max() == 127
    x = synth.bf16_to_f32(synth.normal_bf16(7, 5, (200000,), 0.0, 0.02))
    assert abs(x.std() - 0.02) < 0.0005 and abs(x.mean()) < 0.0005


def test_inventory_matches_pages():
    g = json.load(open(os.path.join(GOLDEN, "qwen3_06b_inventory.json")))
    s = synth.QWEN3_06B
    per_layer = {slot: (int(np.prod(s.matrix_shape(slot))) if slot in synth.MATRIX_SLOTS else s.norm_len(slot))
                 for slot in synth.LAYER_SLOTS}
    n_tensors = 3 + len(synth.LAYER_SLOTS) * s.n_layers          # embed, final norm, lm_head + 11 per block
    embed = s.vocab * s.hidden
    logical = embed + s.hidden + s.n_layers * sum(per_layer.values())
    assert n_tensors == g["tensor_count"]["value"]
    assert embed == g["params_embeddings"]["value"]
    assert logical == g["params_logical"]["value"]
    assert logical + embed == g["params_stored"]["value"]
    assert round(100 * embed / logical, 1) == g["embedding_share_pct_1dp"]["value"]
    assert per_layer["q"] == g["q_proj_params"]["value"]
    assert per_layer["k"] == g["k_proj_params"]["value"]
    assert per_layer["gate"] == g["mlp_proj_params"]["value"]
    kv_f32 = 2 * s.n_layers * s.n_kv_heads * s.head_dim * 8192 * 4
    assert kv_f32 == g["kv_cache_f32_bytes_ctx8192"]["value"]
    # per-layer weight-element formula of the 'Portable WebAssembly Runtime' page (memory accounting)
    D, F = s.hidden, s.inter
    assert D * s.q_dim + 2 * D * s.kv_dim + s.q_dim * D + 3 * D * F == sum(
        v for k, v in per_layer.items() if k in synth.MATRIX_SLOTS)


# ---------------------------------------------------------------------------------------------- storage
def test_bf16_widening_exact_and_rounding_ties_to_even():
    L = oracle.lib()
    for bits in (0x0000, 0x8000, 0x3F80, 0xBF80, 0x7F7F, 0x0001, 0x7F80):
        assert np.float32(L.orc_bf16_to_f32(bits)) == np.array([bits << 16], np.uint32).view(np.float32)[0]
    # 1 + 2^-8 is halfway between bf16 1.0 and 1+2^-7: ties to even -> 1.0
    assert L.orc_f32_to_bf16(1.0 + 2 ** -8) == 0x3F80
    # 1 + 3*2^-8 is halfway between 1+2^-7 (odd) and 1+2^-6 (even) -> rounds up
    assert L.orc_f32_to_bf16(1.0 + 3 * 2 ** -8) == 0x3F82
    assert L.orc_f32_to_bf16(1.0 + 2 ** -8 + 2 ** -20) == 0x3F81


# ---------------------------------------------------------------------------------------------- RMSNorm
def test_rmsnorm_unit_rms_before_scaling():
    rng = np.random.default_rng(0)
    for n in (128, 1024):
        x = rng.standard_normal(n).astype(np.float32) * 3
        out = oracle.rmsnorm(x, np.ones(n, np.float32))
        ms = np.mean(x.astype(np.float64) ** 2)
        rms = math.sqrt(np.mean(out.astype(np.float64) ** 2))
        assert abs(rms - math.sqrt(ms / (ms + 1e-6))) < 1e-6
        w = (1 + 0.1 * rng.standard_normal(n)).astype(np.float32)
        # the weight multiplies the normalised value: one more rounding, elementwise
        assert np.array_equal(oracle.rmsnorm(x, w), (w * out).astype(np.float32))


def test_rmsnorm_constant_vector_closed_form():
    for c in (0.5, 1e-3, 7.0):
        out = oracle.rmsnorm(np.full(64, c, np.float32), np.ones(64, np.float32))
        expect = c / math.sqrt(c * c + 1e-6)
        assert np.allclose(out, expect, rtol=4 * U, atol=0)


# ---------------------------------------------------------------------------------------------- RoPE
def test_rope_position_zero_is_identity():
    c, s = oracle.rope_table(1e6, 128, 0)
    assert np.all(c == 1.0) and np.all(s == 0.0)
    v = np.random.default_rng(1).standard_normal(128).astype(np.float32)
    assert np.array_equal(oracle.rope_apply(v, c, s), v)


def test_rope_preserves_pair_norms_and_composes():
    rng = np.random.default_rng(2)
    v = rng.standard_normal(128).astype(np.float32)
    for pos in (1, 17, 2047, 8191):
        c, s = oracle.rope_table(1e6, 128, pos)
        r = oracle.rope_apply(v, c, s).astype(np.float64)
        n0 = v[:64].astype(np.float64) ** 2 + v[64:].astype(np.float64) ** 2
        n1 = r[:64] ** 2 + r[64:] ** 2
        assert np.max(np.abs(n1 - n0) / n0) < 8 * U
    # R(m) R(n) = R(m + n)
    cm, sm = oracle.rope_table(1e6, 128, 300)
    cn, sn = oracle.rope_table(1e6, 128, 45)
    cmn, smn = oracle.rope_table(1e6, 128, 345)
    two = oracle.rope_apply(oracle.rope_apply(v, cm, sm), cn, sn)
    one = oracle.rope_apply(v, cmn, smn)
    assert np.max(np.abs(two - one)) < 1e-5


def test_rope_inner_product_depends_on_offset_only():
    rng = np.random.default_rng(3)
    q = rng.standard_normal(128).astype(np.float32)
    k = rng.standard_normal(128).astype(np.float32)
    vals = []
    for m in (3, 103, 1003, 5003):
        rq = oracle.rope_apply(q, *oracle.rope_table(1e6, 128, m + 7))
        rk = oracle.rope_apply(k, *oracle.rope_table(1e6, 128, m))
        vals.append(float(np.dot(rq.astype(np.float64), rk.astype(np.float64))))
    assert max(vals) - min(vals) < 2e-4


def test_rope_alternating_vector_large_position():
    """Hand-check vector of section 9 ('RoPE Extreme Boundaries'): alternating ones and zeros at a large
    position.  Low pair indices rotate by large angles, the highest ones barely move; values agree with
    an independent fp64 evaluation and with HF transformers' rotary helper (rotate-half pairing)."""
    import torch
    from transformers.models.qwen3.modeling_qwen3 import apply_rotary_pos_emb

    v = np.tile(np.array([1.0, 0.0], np.float32), 64)
    pos = 8000
    c, s = oracle.rope_table(1e6, 128, pos)
    r = oracle.rope_apply(v, c, s)
    ref64 = twin64.rope64(v.astype(np.float64)[None, :], [pos], 1e6)[0]
    assert np.max(np.abs(r - ref64)) < 1e-6
    moved = np.abs(r - v)
    assert moved[62] < 0.02 and moved[126] < 0.02          # lowest frequency pair (62, 126)
    assert moved[:8].max() > 0.5                           # fastest pairs swing hard
    cc = torch.from_numpy(np.concatenate([c, c]).astype(np.float64))[None, None]
    ss = torch.from_numpy(np.concatenate([s, s]).astype(np.float64))[None, None]
    t = torch.from_numpy(v.astype(np.float64))[None, None, None]
    hf, _ = apply_rotary_pos_emb(t, t, cc, ss)
    assert np.max(np.abs(hf.numpy().reshape(-1) - r)) < 1e-6


# ---------------------------------------------------------------------------------------------- softmax
def test_softmax_cases():
    rc, p = oracle.softmax(np.array([3.5], np.float32))
    assert rc == 0 and p[0] == 1.0
    rc, _ = oracle.softmax(np.array([], np.float32))
    assert rc == oracle.ORC_INVALID_ARGUMENT
    rc, _ = oracle.softmax(np.array([1.0, np.nan], np.float32))
    assert rc == oracle.ORC_NUMERICAL_FAILURE
    rng = np.random.default_rng(4)
    for n in (2, 37, 4096):
        s = (rng.standard_normal(n) * 5).astype(np.float32)
        rc, p = oracle.softmax(s)
        assert rc == 0 and abs(float(np.sum(p.astype(np.float64))) - 1.0) <= n * U
        rc, p2 = oracle.softmax(s + np.float32(64.0))       # max-shift invariance
        assert np.max(np.abs(p2 - p)) < 1e-5
    rc, p = oracle.softmax(np.array([1000.0, 999.0], np.float32))    # no overflow; closed form
    assert rc == 0 and abs(p[0] - 1 / (1 + math.exp(-1))) < 2e-7


# ---------------------------------------------------------------------------------------------- attention
def test_attention_single_cached_token_returns_v_exactly():
    rng = np.random.default_rng(5)
    q = rng.standard_normal(128).astype(np.float32)
    k = rng.standard_normal((1, 128)).astype(np.float32)
    v = rng.standard_normal((1, 128)).astype(np.float32)
    rc, out = oracle.attention_head(q, k, v)
    assert rc == 0 and np.array_equal(out, v[0])


def test_attention_zero_query_is_mean_of_v():
    rng = np.random.default_rng(6)
    v = rng.standard_normal((50, 128)).astype(np.float32)
    k = rng.standard_normal((50, 128)).astype(np.float32)
    rc, out = oracle.attention_head(np.zeros(128, np.float32), k, v)
    assert rc == 0 and np.max(np.abs(out - v.astype(np.float64).mean(0))) < 1e-5


def test_attention_matches_softmax_brute_force():
    rng = np.random.default_rng(7)
    n, d = 33, 128
    q = rng.standard_normal(d).astype(np.float32)
    k = rng.standard_normal((n, d)).astype(np.float32)
    v = rng.standard_normal((n, d)).astype(np.float32)
    rc, out = oracle.attention_head(q, k, v)
    s = k.astype(np.float64) @ q.astype(np.float64) / math.sqrt(d)
    p = np.exp(s - s.max())
    p /= p.sum()
    assert rc == 0 and np.max(np.abs(out - p @ v.astype(np.float64))) < 1e-5


def test_gqa_head_routing():
    """Section 9 'GQA Head Mapping Routing': 4 query heads over 2 KV heads; KV head 0 carries large
    positive identifiers and head 1 large negative ones; query heads 2 and 3 must see only head 1."""
    rng = np.random.default_rng(8)
    n, d = 6, 128
    ident = np.arange(1, n + 1, dtype=np.float32)[:, None] * np.ones((1, d), np.float32)
    k = np.stack([1000 + ident, -1000 - ident]) / 1000
    v = np.stack([1000 + ident, -1000 - ident])
    q = rng.standard_normal((4, d)).astype(np.float32)
    rc, out = oracle.gqa_attention(q, k, v)
    assert rc == 0
    assert np.all(out[:2] >= 1000) and np.all(out[2:] <= -1000)
    for h in range(4):
        _, ref = oracle.attention_head(q[h], k[h // 2], v[h // 2])
        assert np.array_equal(out[h], ref)
    rc, _ = oracle.gqa_attention(q[:3], k, v)               # 3 % 2 != 0
    assert rc == oracle.ORC_INVALID_ARGUMENT


# ---------------------------------------------------------------------------------------------- SwiGLU
def test_silu_cases():
    """Section 9 'Adversarial SwiGLU': silu(0)=0, saturation to the identity for large z, and a tiny
    negative (not zero) output for strongly negative z."""
    assert oracle.silu(0.0) == 0.0
    for z in (17.0, 20.0, 88.0):
        assert oracle.silu(z) == np.float32(z)
    for z in (-20.0, -5.0, -1.0, 0.5, 3.0):
        exact = z / (1 + math.exp(-z))
        got = float(oracle.silu(z))
        assert abs(got - exact) <= 4 * U * abs(exact)
    assert -1e-7 < oracle.silu(-20.0) < 0.0


# ---------------------------------------------------------------------------------------------- Q8
def test_q8_dequant_is_one_f32_multiply_and_round_trips():
    codes = np.arange(-127, 128, dtype=np.int8)
    for s in np.float32([1e-3, 3.7e-3, 1e-2, 0.5, 1.0]):
        deq = codes.astype(np.float32) * s            # IEEE f32 product
        m = synth.Matrix(1, 32, codes=np.resize(codes, 32)[None].copy(), scales=np.array([[s]], np.float32))
        assert np.array_equal(oracle.dequant_row(m, 0), np.resize(codes, 32).astype(np.float32) * s)
        assert np.array_equal(np.rint(deq / s).astype(np.int8), codes)


def test_q8_quantized_tail_vector_sums_to_zero():
    """Section 9 'Quantized Tails': one 32-block alternating +127/-127 with unit activations."""
    codes = np.tile(np.array([127, -127], np.int8), 16)
    for s in (np.float32(7e-3), np.float32(1.0), np.float32(2.0 ** -130)):   # last one is subnormal-scaled
        assert oracle.q8_dot(codes, np.array([s], np.float32), np.ones(32, np.float32)) == 0.0


@pytest.mark.parametrize("fmt", [synth.FMT_BF16, synth.FMT_Q8])
def test_matvec_within_summation_bound(fmt):
    shp = replace(TINY, fmt=fmt, hidden=256)
    m = synth._matrix(shp, 9, 42, 40, 256, 0.02)
    x = np.random.default_rng(9).standard_normal(256).astype(np.float32)
    y = oracle.matvec(m, x)
    w64 = twin64._mat64(m)
    prods = np.abs(w64 * x.astype(np.float64)[None, :]).sum(1)
    exact = w64 @ x.astype(np.float64)
    extra = 1 if fmt == synth.FMT_BF16 else 2               # q*s then act*(q*s): one more rounding
    assert np.all(np.abs(y - exact) <= gamma(256 + extra) * prods)


def test_argmax_ties_and_non_finite():
    rc, i = oracle.argmax(np.array([1.0, 5.0, 2.0, 5.0, 5.0], np.float32))
    assert rc == 0 and i == 1
    rc, _ = oracle.argmax(np.array([1.0, np.nan, 2.0], np.float32))
    assert rc == oracle.ORC_NUMERICAL_FAILURE
    rc, _ = oracle.argmax(np.array([1.0, np.inf], np.float32))
    assert rc == oracle.ORC_NUMERICAL_FAILURE


# ---------------------------------------------------------------------------------------------- model
@pytest.mark.parametrize("fmt", [synth.FMT_BF16, synth.FMT_Q8])
@pytest.mark.parametrize("kv_f32", [True, False])
def test_model_matches_fp64_twin(fmt, kv_f32):
    shp = replace(TINY, fmt=fmt)
    W = synth.make_weights(shp, seed=11)
    toks = synth.tokens(11, 0, 8, shp.vocab)
    m = oracle.Model(W, kv_f32=kv_f32)
    rc, am, lg = m.prefill(toks)
    _, ref = twin64.forward64(W, tokens=toks, kv_round_bf16=not kv_f32)
    assert rc == 0
    assert np.max(np.abs(lg - ref)) <= 1e-5 * np.max(np.abs(ref))
    assert am == int(np.argmax(ref))


def test_single_block_real_dims_matches_fp64_twin():
    """One real-width Qwen3-0.6B block (hidden 1024, 16/8 heads of 128, MLP 3072) on fp32 hidden inputs."""
    shp = replace(synth.SINGLE_BLOCK.shape, max_ctx=16)
    W = synth.make_weights(shp, seed=1)
    hin = synth.hidden_inputs(1, 0, 6, shp.hidden)
    m = oracle.Model(W, kv_f32=True)
    outs = [m.step(0, hidden_in=hin[t], want_hidden=True)[3] for t in range(6)]
    ref, _ = twin64.forward64(W, hidden=hin)
    err = np.max(np.abs(np.stack(outs) - ref))
    assert err <= 1e-5 * np.max(np.abs(ref))


def _hf_model(W):
    import torch
    from transformers import Qwen3Config, Qwen3ForCausalLM
    s = W.shape
    cfg = Qwen3Config(vocab_size=s.vocab, hidden_size=s.hidden, intermediate_size=s.inter,
                      num_hidden_layers=s.n_layers, num_attention_heads=s.n_q_heads,
                      num_key_value_heads=s.n_kv_heads, head_dim=s.head_dim, rms_norm_eps=s.eps,
                      rope_theta=s.theta, tie_word_embeddings=True, max_position_embeddings=64,
                      attention_bias=False, hidden_act="silu")
    model = Qwen3ForCausalLM(cfg).double().eval()
    f = lambda m: torch.from_numpy(twin64._mat64(m)) if hasattr(m, "is_q8") else torch.from_numpy(
        twin64._norm64(m, s.fmt))
    names = {"attn_norm": "input_layernorm", "q": "self_attn.q_proj", "k": "self_attn.k_proj",
             "v": "self_attn.v_proj", "q_norm": "self_attn.q_norm", "k_norm": "self_attn.k_norm",
             "o": "self_attn.o_proj", "mlp_norm": "post_attention_layernorm", "gate": "mlp.gate_proj",
             "up": "mlp.up_proj", "down": "mlp.down_proj"}
    sd = {"model.embed_tokens.weight": f(W.embed), "model.norm.weight": f(W.final_norm)}
    for l, d in enumerate(W.layers):
        for k, v in d.items():
            sd[f"model.layers.{l}.{names[k]}.weight"] = f(v)
    sd["lm_head.weight"] = sd["model.embed_tokens.weight"]
    res = model.load_state_dict(sd, strict=False)
    assert not res.missing_keys and not res.unexpected_keys
    return model


@pytest.mark.parametrize("fmt", [synth.FMT_BF16, synth.FMT_Q8])
def test_model_matches_hf_qwen3(fmt):
    """The pages name the PyTorch Qwen3 model as the conformance reference (section 10); HF transformers'
    Qwen3ForCausalLM in fp64 on the same tiny weights pins RoPE pairing, QK-Norm placement, the GQA map,
    SwiGLU and the tied logits."""
    import torch
    shp = replace(TINY, fmt=fmt)
    W = synth.make_weights(shp, seed=12)
    toks = synth.tokens(12, 0, 9, shp.vocab)
    with torch.no_grad():
        ref = _hf_model(W)(torch.from_numpy(toks.astype(np.int64))[None]).logits[0, -1].numpy()
    m = oracle.Model(W, kv_f32=True)
    rc, am, lg = m.prefill(toks)
    assert rc == 0
    assert np.max(np.abs(lg - ref)) <= 1e-5 * np.max(np.abs(ref))
    assert am == int(np.argmax(ref))


def test_thread_count_does_not_change_bits():
    W = synth.make_weights(replace(TINY, fmt=synth.FMT_Q8), seed=13)
    toks = synth.tokens(13, 0, 5, TINY.vocab)
    n0 = oracle.get_threads()
    try:
        oracle.set_threads(1)
        _, a1, l1 = oracle.Model(W).prefill(toks)
        oracle.set_threads(max(2, n0))
        _, a2, l2 = oracle.Model(W).prefill(toks)
    finally:
        oracle.set_threads(n0)
    assert a1 == a2 and np.array_equal(l1, l2)


def test_context_overflow_is_typed_and_leaves_state():
    shp = replace(TINY, max_ctx=4)
    W = synth.make_weights(shp, seed=14)
    m = oracle.Model(W)
    toks = synth.tokens(14, 0, 4, shp.vocab)
    rc, _, _ = m.prefill(toks)
    assert rc == 0 and m.get_len(0) == 4
    _, k0, v0 = m.kv_read(0, 1, 0, 4)
    rc, *_ = m.step(0, 3)
    assert rc == oracle.ORC_CONTEXT_EXCEEDED and m.get_len(0) == 4
    _, k1, v1 = m.kv_read(0, 1, 0, 4)
    assert np.array_equal(k0, k1) and np.array_equal(v0, v1)


def test_reset_then_replay_equals_fresh_and_kv_roundtrip():
    W = synth.make_weights(TINY, seed=15)
    toks = synth.tokens(15, 0, 6, TINY.vocab)
    m = oracle.Model(W)
    _, a1, l1 = m.prefill(toks)
    m.set_len(0, 0)                     # reset: length only, cache bytes left in place
    _, a2, l2 = m.prefill(toks)
    assert a1 == a2 and np.array_equal(l1, l2)
    k, v = synth.kv_fill(15, 0, 1, TINY.n_kv_heads, 5, TINY.head_dim)
    assert m.kv_write(0, 1, 3, k, v) == 0
    rc, k2, v2 = m.kv_read(0, 1, 3, 5)
    assert rc == 0 and np.array_equal(k, k2) and np.array_equal(v, v2)
    assert m.kv_write(0, 1, TINY.max_ctx - 2, k, v) == oracle.ORC_INVALID_ARGUMENT



# ---------------------------------------------------------------------------------------------------------
# Q8_0 blocks ("Scalar-Native ...", section 3 "The Q8_0 Block Contract", section 5 q8_dot, section 9
# "Quantized Tails")
# ---------------------------------------------------------------------------------------------------------
def test_f16_to_f32_every_bit_pattern():
    """The oracle's binary16 widening, written from the format definition, against numpy's IEEE half type for
    all 65,536 patterns (NaN patterns must stay NaN)."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = np.array([oracle.f16_to_f32(b) for b in bits], np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def _block(scale16_bits, codes):
    return np.concatenate([np.array([scale16_bits & 0xFF, scale16_bits >> 8], np.uint8),
                           np.asarray(codes, np.int8).view(np.uint8)])


@pytest.mark.parametrize("scale_bits", [0x0001, 0x03FF, 0x0400, 0x3C00, 0x7BFF])
def test_q8_0_quantized_tails_vector(scale_bits):
    """Section 9's vector: one block whose payload alternates the extremes +127/-127, against ones.  Every
    product q * scale is exact in f32 even for a subnormal f16 scale (2^-24 * 127 is a normal f32), so the
    sequential sum returns to exactly 0 after each pair: the result is exactly 0, with no underflow."""
    codes = np.array([127, -127] * 16, np.int8)
    assert oracle.q8_0_dot(_block(scale_bits, codes), np.ones(32, np.float32)) == 0.0
    # and a constant payload gives exactly 32 * q * scale (every partial sum is a small multiple of q * s)
    s = float(np.array([scale_bits], np.uint16).view(np.float16)[0])
    got = oracle.q8_0_dot(_block(scale_bits, np.full(32, 5, np.int8)), np.ones(32, np.float32))
    assert got == np.float32(np.float32(5.0) * np.float32(s)) * 32


def test_q8_0_dot_follows_the_page_order_and_equals_widened_q8():
    """The block reader against the pages' loop evaluated in numpy f32 step by step, and against the f32-scale
    Q8 dot with the scales widened (identical arithmetic once the f16 scale is read)."""
    rng = np.random.default_rng(7)
    n = 1024
    codes = rng.integers(-127, 128, n).astype(np.int8)
    scales16 = rng.uniform(1e-3, 1e-2, n // 32).astype(np.float16)
    act = rng.standard_normal(n).astype(np.float32)
    m = synth.q8_0_matrix(codes.reshape(1, n), scales16.reshape(1, -1))
    got = oracle.q8_0_dot(m.q8_0[0], act)
    acc = np.float32(0)
    for b in range(n // 32):
        sc = np.float32(scales16[b])
        for i in range(32):
            acc = np.float32(acc + np.float32(act[32 * b + i] * np.float32(np.float32(codes[32 * b + i]) * sc)))
    assert got == acc
    assert got == oracle.q8_dot(codes, scales16.astype(np.float32), act)


def test_q8_0_round_trip_and_dequant():
    """Dequantized element = one f32 multiply of the code by the widened f16 scale; re-quantizing with that
    scale returns every code in [-127, 127]."""
    shp = replace(synth.QWEN3_06B, fmt=synth.FMT_Q8_0, vocab=64, n_layers=1, hidden=1024, inter=1024,
                  n_q_heads=8, n_kv_heads=4)
    W = synth.make_weights(shp, seed=3)
    m = W.layers[0]["o"]
    for r in (0, 17, m.rows - 1):
        row = oracle.dequant_row(m, r)
        sc = np.repeat(m.scales[r], 32)
        assert np.array_equal(row.view(np.uint32), (m.codes[r].astype(np.float32) * sc).view(np.uint32))
        assert np.array_equal(np.rint(row / sc).astype(np.int32), m.codes[r].astype(np.int32))


def test_q8_0_model_equals_widened_q8_model():
    """A whole Q8_0 model through the oracle gives bit-identical logits to the same model given as codes plus
    the widened scales (the block format changes storage, not arithmetic), and agrees with the fp64 twin."""
    shp = replace(TINY, fmt=synth.FMT_Q8_0)
    W = synth.make_weights(shp, seed=12)
    toks = synth.tokens(12, 0, 6, shp.vocab)
    a = oracle.Model(W)
    # the same codes and widened scales without the blocks: the oracle reads them as the f32-scale format
    plain = lambda m: synth.Matrix(m.rows, m.cols, codes=m.codes, scales=m.scales)
    W8 = synth.Weights(replace(shp, fmt=synth.FMT_Q8), plain(W.embed), W.final_norm,
                       [{k: (plain(v) if isinstance(v, synth.Matrix) else v) for k, v in d.items()} for d in W.layers])
    b = oracle.Model(W8)
    for t in toks:
        ra, _, la, _ = a.step(0, int(t))
        rb, _, lb, _ = b.step(0, int(t))
        assert ra == rb == 0 and np.array_equal(la.view(np.uint32), lb.view(np.uint32))
    _, l64 = twin64.forward64(W, tokens=toks, kv_round_bf16=True)
    assert np.max(np.abs(la - l64)) / np.max(np.abs(l64)) < 1e-4


def test_step_with_its_own_kv_forced_is_the_plain_step():
    """Teacher forcing of the appended position: a step that reports its own rounded K/V gives the plain step's
    logits bit for bit and caches exactly those values; a forced value is what the cache then holds."""
    W = synth.make_weights(replace(TINY, fmt=synth.FMT_Q8), seed=13)
    a, b = oracle.Model(W), oracle.Model(W)
    toks = synth.tokens(13, 0, 5, TINY.vocab)
    for i, t in enumerate(toks):
        ra, _, la, _ = a.step(0, int(t))
        rb, _, lb, _, own = b.step_forced(0, int(t))
        assert ra == rb == 0 and np.array_equal(la.view(np.uint32), lb.view(np.uint32))
        _, k, v = b.kv_read(0, 1, i, 1)
        assert np.array_equal(k[:, 0], own[1, 0]) and np.array_equal(v[:, 0], own[1, 1])
    c = oracle.Model(W)
    forced = own.copy()
    forced[0, 1, 0, 3] ^= 1
    assert c.step_forced(0, int(toks[0]), kv_force=forced)[0] == 0
    _, k, v = c.kv_read(0, 0, 0, 1)
    assert v[0, 0, 3] == forced[0, 1, 0, 3] and np.array_equal(k[:, 0], forced[0, 0])


# ---------------------------------------------------------------------------------------------------------
# q8 x q8 with dynamically quantized int8 activations ("Real-Browser WASM Qwen3 Execution ...", section 5
# "Q8_0 Mixed-Precision Matrix Multiplication"; "Portable WebAssembly ...", "Integer-overflow rule")
# ---------------------------------------------------------------------------------------------------------
def test_act8_block_scale_and_ties_away_from_zero():
    """A block whose largest magnitude is 127 has scale 1, so the codes are the inputs rounded to nearest
    with ties away from zero (0.5 -> 1, 2.5 -> 3, -0.5 -> -1), not to even."""
    x = np.zeros(32, np.float32)
    x[:8] = [127.0, 0.5, 1.5, 2.5, -0.5, -2.5, 3.49, -126.6]
    q, d = oracle.quantize_act8(x)
    assert d[0] == 1.0
    assert list(q[:8]) == [127, 1, 2, 3, -1, -3, 3, -127]
    assert np.all(q[8:] == 0)


def test_act8_codes_on_the_grid_round_trip_and_rounding_bound():
    rng = np.random.default_rng(11)
    codes = rng.integers(-127, 128, 64).astype(np.int8)
    codes[0], codes[32] = 127, -127                          # each block reaches the bound
    d = np.array([0.037, 1e-30], np.float32)                  # a normal and a tiny scale
    x = (codes.astype(np.float32) * np.repeat(d, 32)).astype(np.float32)
    q, dd = oracle.quantize_act8(x)
    assert np.array_equal(q, codes)
    y = (3 * rng.standard_normal(4096)).astype(np.float32)
    q, dd = oracle.quantize_act8(y)
    err = np.abs(q.astype(np.float64) * np.repeat(dd.astype(np.float64), 32) - y)
    assert np.all(err <= np.repeat(dd, 32) * 0.5 * (1 + 1e-6)) and np.all(np.abs(q) <= 127)


def test_act8_zero_and_non_finite_blocks():
    x = np.zeros(64, np.float32)
    x[40] = np.nan
    q, d = oracle.quantize_act8(x)
    assert d[0] == 0.0 and np.all(q[:32] == 0)
    assert np.isnan(d[1]) and np.all(q[32:] == 0)            # the NaN stays in the scale, codes are inert
    w = np.ones(64, np.int8)
    assert oracle.q8q8_dot(w, np.ones(2, np.float32), q, d) != oracle.q8q8_dot(w, np.ones(2, np.float32), q, d)


def test_q8q8_dot_integer_bound_and_exact_block_sums():
    """The worst block, all codes +-127 on both sides, sums to 32 * 127 * 127 = 516,128 (< 2^31 - 1, the
    integer-overflow rule), exactly; with scales that are powers of two the whole dot is exact."""
    assert 32 * 127 * 127 == 516128 < 2 ** 31 - 1
    w = np.full(64, -127, np.int8)
    a = np.full(64, -127, np.int8)
    a[32:] = 127
    got = oracle.q8q8_dot(w, np.array([0.5, 0.25], np.float32), a, np.array([2.0, 4.0], np.float32))
    assert got == 516128 * 1.0 - 516128 * 1.0
    a[:] = 127
    assert oracle.q8q8_dot(w, np.array([0.5, 0.25], np.float32), a, np.array([2.0, 4.0], np.float32)) == -2 * 516128.0


def test_q8q8_dot_equals_fp64_of_the_quantized_values():
    """Against the exact fp64 dot of the dequantized weights and the dequantized activation codes, within the
    f32 summation bound over the blocks."""
    rng = np.random.default_rng(12)
    n = 1024
    wq = rng.integers(-127, 128, n).astype(np.int8)
    ws = rng.uniform(1e-3, 1e-2, n // 32).astype(np.float32)
    x = rng.standard_normal(n).astype(np.float32)
    aq, ad = oracle.quantize_act8(x)
    got = float(oracle.q8q8_dot(wq, ws, aq, ad))
    terms = [float(np.dot(wq[32 * b:32 * b + 32].astype(np.int64), aq[32 * b:32 * b + 32].astype(np.int64)))
             * float(ws[b]) * float(ad[b]) for b in range(n // 32)]
    exact = sum(terms)
    nb = n // 32
    gamma = (nb + 2) * 2.0 ** -24 / (1 - (nb + 2) * 2.0 ** -24)
    assert abs(got - exact) <= gamma * sum(abs(t) for t in terms)


def test_act8_model_tracks_the_f32_activation_model():
    """The whole model in the q8 x q8 format against the same weights with f32 activations: the logits differ
    by the activation quantization error only (small but not zero), and every step stays finite."""
    shp = replace(TINY, fmt=synth.FMT_Q8_ACT8)
    W = synth.make_weights(shp, seed=14)
    Wf = synth.Weights(replace(shp, fmt=synth.FMT_Q8), W.embed, W.final_norm, W.layers)
    a, b = oracle.Model(W), oracle.Model(Wf)
    for t in synth.tokens(14, 0, 6, shp.vocab):
        ra, _, la, _ = a.step(0, int(t))
        rb, _, lb, _ = b.step(0, int(t))
        assert ra == rb == 0
        r = np.linalg.norm(la - lb) / np.linalg.norm(lb)
        assert 1e-5 < r < 5e-2, r
