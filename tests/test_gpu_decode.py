"""GPU parity of the decode path against the oracle (through the C ABI).

Shapes: real-width blocks (hidden 1024, head_dim 128) with few layers and a ragged vocabulary (1000 rows:
not a multiple of any GEMV tile), plus the GQA group sizes the kernels support, at sizes the oracle
finishes in seconds.
"""
import sys
from dataclasses import replace

import numpy as np
import pytest

import oracle
import synth
from parity import (ACT8_COS, ACT8_KV_REL, Margins, argmax_ok, assert_close, build_gpu_model, cosine, forced_step,
                    forced_step_act8, rel_l2)

pytestmark = pytest.mark.gpu

SMALL = replace(synth.QWEN3_06B, vocab=1000, n_layers=2, n_q_heads=8, n_kv_heads=4, inter=1024, max_ctx=64,
                max_prefill=32)


def _torch():
    import torch
    assert torch.cuda.is_available()
    return torch


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("fmt", [synth.FMT_BF16, synth.FMT_Q8, synth.FMT_Q8_0])
def test_dequant_bit_exact(fmt):
    torch = _torch()
    shp = replace(SMALL, fmt=fmt)
    _say("dequant", shp)
    W = synth.make_weights(shp, seed=21)
    m = build_gpu_model(W)
    for kind, layer in (("q", 0), ("k", 1), ("v", 1), ("o", 0), ("gate", 1), ("up", 0), ("down", 1),
                        ("embed", -1)):
        mat = W.embed if kind == "embed" else W.layers[layer][kind]
        got = m.dequant(kind, layer, mat.rows, mat.cols).cpu().numpy()
        torch.cuda.synchronize()
        rows = np.arange(mat.rows)
        ref = np.stack([oracle.dequant_row(mat, r) for r in rows])
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), kind


def test_kv_write_read_roundtrip_and_bounds():
    torch = _torch()
    m = build_gpu_model(synth.make_weights(SMALL, seed=22))
    k, v = synth.kv_fill(22, 0, 1, SMALL.n_kv_heads, 7, SMALL.head_dim)
    kt = torch.from_numpy(k.view(np.int16)).cuda()
    vt = torch.from_numpy(v.view(np.int16)).cuda()
    m.kv_write(0, 1, 5, kt, vt)
    k2, v2 = m.kv_read(0, 1, 5, 7)
    assert np.array_equal(k2.cpu().numpy().view(np.uint16), k)
    assert np.array_equal(v2.cpu().numpy().view(np.uint16), v)
    import transformer_qwen3_block_amd as q
    with pytest.raises(q.Qw3Error) as e:
        m.kv_write(0, 1, SMALL.max_ctx - 3, kt, vt)
    assert e.value.code == 6


def _build(W, path):
    """path "mega": single-sequence steps as one persistent launch (the default where the shape allows);
    "kernels": one launch per step of the layer (QW3_NO_MEGA=1 at creation)."""
    import os
    if path == "kernels":
        os.environ["QW3_NO_MEGA"] = "1"
    try:
        return build_gpu_model(W)
    finally:
        os.environ.pop("QW3_NO_MEGA", None)


def _greedy_vs_oracle(shp, seed, steps, prefill_tokens=0, kv_fill_len=0, seqs_checked=None, path="mega"):
    """Free-running GPU greedy decode, replayed through the oracle (teacher forcing)."""
    torch = _torch()
    W = synth.make_weights(shp, seed=seed)
    m = _build(W, path)
    S = shp.n_seq
    orc = oracle.Model(W)
    if kv_fill_len:
        for s in range(S):
            for l in range(shp.n_layers):
                k, v = synth.kv_fill(seed, s, l, shp.n_kv_heads, kv_fill_len, shp.head_dim)
                m.kv_write(s, l, 0, torch.from_numpy(k.view(np.int16)).cuda(),
                           torch.from_numpy(v.view(np.int16)).cuda())
                orc.kv_write(s, l, 0, k, v)
            m.set_len(s, kv_fill_len)
            orc.set_len(s, kv_fill_len)
    toks = synth.tokens(seed, 1, S, shp.vocab)
    cur = torch.from_numpy(toks.copy()).cuda()
    am = torch.empty(S, dtype=torch.int32, device="cuda")
    logits = torch.empty((S, shp.vocab), dtype=torch.float32, device="cuda")
    worst = Margins(f"decode {shp.fmt=} {shp.n_layers=} {shp.n_q_heads}/{shp.n_kv_heads} heads S={S} {path}")
    kv = {}
    act8 = shp.fmt == synth.FMT_Q8_ACT8   # q8 x q8: greedy agreement and logits cosine per step
    worst_cos, worst_abs, worst_rel = 1.0, 0.0, 0.0
    for step in range(steps):
        m.decode_step(cur, am, logits)
        torch.cuda.synchronize()
        g_logits = logits.cpu().numpy()
        g_am = am.cpu().numpy()
        for s in (seqs_checked if seqs_checked is not None else range(S)):
            if act8:
                rc, o_am, o_logits, _ = forced_step_act8(m, orc, s, int(cur[s].item()), shp.n_layers, stats=kv)
                assert rc == 0
                c = cosine(g_logits[s], o_logits)
                worst_cos = min(worst_cos, c)
                d = np.abs(g_logits[s].astype(np.float64) - o_logits)
                worst_abs, worst_rel = max(worst_abs, float(d.max())), max(worst_rel, rel_l2(g_logits[s], o_logits))
                assert c >= ACT8_COS, f"step {step} seq {s}: logits cosine {c:.6f}"
            else:
                rc, o_am, o_logits, _ = forced_step(m, orc, s, int(cur[s].item()), shp.n_layers, stats=kv)
                assert rc == 0
                worst.add(assert_close(g_logits[s], o_logits, f"step {step} seq {s}"))
            assert argmax_ok(int(g_am[s]), o_logits, g_logits[s]), (step, s, int(g_am[s]), o_am)
        cur = am.clone()
    assert m.status() == 0
    for s in range(S):
        assert m.get_len(s) == kv_fill_len + steps
    if act8:
        _say(f"MARGIN q8 x q8 decode {shp.n_layers} layer(s) {shp.n_q_heads}/{shp.n_kv_heads} heads: worst logits "
             f"cosine {worst_cos:.6f} (bound {ACT8_COS}); for information worst max-abs {worst_abs:.3e}, worst "
             f"rel-L2 {worst_rel:.3e}, worst appended K/V rel-L2 {kv.get('kv_rel', 0):.3e} (bound {ACT8_KV_REL})")
        return None
    worst.report(kv)
    return worst


@pytest.mark.parametrize("path", ["mega", "kernels"])
@pytest.mark.parametrize("fmt", [synth.FMT_BF16, synth.FMT_Q8, synth.FMT_Q8_0])
def test_decode_small_vs_oracle(fmt, path):
    shp = replace(SMALL, fmt=fmt)
    _say("decode small", shp, path)
    _greedy_vs_oracle(shp, seed=23, steps=12, path=path)


@pytest.mark.parametrize("path", ["mega", "kernels"])
@pytest.mark.parametrize("heads", [(8, 8), (8, 2), (16, 4)])
def test_decode_gqa_group_sizes(heads, path):
    shp = replace(SMALL, n_q_heads=heads[0], n_kv_heads=heads[1], n_layers=1)
    _say("gqa", heads, path)
    _greedy_vs_oracle(shp, seed=24, steps=6, path=path)


@pytest.mark.parametrize("path", ["mega", "kernels"])
def test_decode_over_prefilled_cache_ragged_context(path):
    """Context lengths that are not multiples of the 16-position groups or of the split count."""
    shp = replace(SMALL, fmt=synth.FMT_Q8, max_ctx=400)
    _say("ragged context", path)
    _greedy_vs_oracle(shp, seed=25, steps=4, kv_fill_len=333, path=path)


def test_decode_uneven_position_split_long_context():
    """Eight KV heads over 2301 cached positions: 576 four-position quads over 128 wave slots per KV head, so
    half the slots take five quads (one whole five-quad chunk) and the rest four."""
    shp = replace(SMALL, fmt=synth.FMT_Q8, n_q_heads=16, n_kv_heads=8, n_layers=1, max_ctx=2400)
    _say("uneven split", shp)
    _greedy_vs_oracle(shp, seed=27, steps=3, kv_fill_len=2301, path="mega")


@pytest.mark.parametrize("heads,ctx", [((16, 8), 6000), ((16, 4), 4200)])
def test_decode_long_context_several_chunks(heads, ctx):
    """Contexts long enough that every wave slot walks several attention chunks, the next chunk's K/V in flight
    while the current one is scored: 6000 positions over 128 wave slots of a KV head (about 12 quads each:
    passes of five, five and two) with two query heads per KV head, and 4200 positions over 256 slots (four-quad
    chunks) with four."""
    shp = replace(SMALL, fmt=synth.FMT_Q8, n_q_heads=heads[0], n_kv_heads=heads[1], n_layers=1, max_ctx=ctx + 8)
    _say("long context", heads, ctx)
    _greedy_vs_oracle(shp, seed=41, steps=3, kv_fill_len=ctx, path="mega")


def test_decode_batched_sequences():
    shp = replace(SMALL, fmt=synth.FMT_Q8, n_seq=5, max_ctx=200)
    _greedy_vs_oracle(shp, seed=26, steps=3, kv_fill_len=150)


@pytest.mark.parametrize("n_seq,heads,inter", [(2, (8, 4), 1024), (16, (8, 4), 1024), (3, (16, 8), 3072)])
def test_decode_batched_q8_mfma_shapes(n_seq, heads, inter):
    """Batched Q8 steps take the MFMA products: 2 and 16 sequences (the extremes of the 16-wide tiles) and
    the full-size projection shapes (q_dim 2048, intermediate 3072) at two layers."""
    shp = replace(SMALL, fmt=synth.FMT_Q8, n_seq=n_seq, n_q_heads=heads[0], n_kv_heads=heads[1], inter=inter,
                  max_ctx=96)
    _say("batched q8 mfma", n_seq, heads, inter)
    _greedy_vs_oracle(shp, seed=28, steps=3, kv_fill_len=40, seqs_checked=(0, n_seq - 1))


def test_context_exceeded_leaves_state():
    torch = _torch()
    import transformer_qwen3_block_amd as q
    shp = replace(SMALL, max_ctx=3)
    m = build_gpu_model(synth.make_weights(shp, seed=27))
    cur = torch.zeros(1, dtype=torch.int32, device="cuda")
    am = torch.empty(1, dtype=torch.int32, device="cuda")
    for _ in range(3):
        m.decode_step(cur, am)
    with pytest.raises(q.Qw3Error) as e:
        m.decode_step(cur, am)
    assert e.value.code == 14 and m.get_len(0) == 3
    m.reset_kv(0)
    assert m.get_len(0) == 0
    m.decode_step(cur, am)
    torch.cuda.synchronize()
    assert m.get_len(0) == 1 and m.status() == 0


def test_single_block_decode_hidden_states():
    """Single real-size block in hidden-state mode, one position at a time."""
    torch = _torch()
    shp = replace(synth.SINGLE_BLOCK.shape)
    W = synth.make_weights(shp, seed=1)
    m = build_gpu_model(W)
    orc = oracle.Model(W)
    hin = synth.hidden_inputs(1, 1, 8, shp.hidden)
    out = torch.empty((1, shp.hidden), dtype=torch.float32, device="cuda")
    for t in range(8):
        m.block_forward(torch.from_numpy(hin[t:t + 1]).cuda(), out)
        torch.cuda.synchronize()
        rc, _, _, ref = orc.step(0, hidden_in=hin[t], want_hidden=True)
        assert rc == 0
        assert_close(out.cpu().numpy()[0], ref, f"position {t}")


def test_graph_replay_matches_eager_bitwise():
    """Decode steps replayed from a captured HIP graph (side stream) equal eager launches (null stream) bit
    for bit, over several replays with host work and synchronisations between them."""
    torch = _torch()
    import os
    shp = replace(SMALL, fmt=synth.FMT_Q8, max_ctx=64)
    W = synth.make_weights(shp, seed=28)
    os.environ["QW3_NO_GRAPH"] = "1"
    try:
        eager = build_gpu_model(W)
    finally:
        del os.environ["QW3_NO_GRAPH"]
    graphed = build_gpu_model(W)
    side = torch.cuda.Stream()
    tok0 = torch.tensor(synth.tokens(28, 1, 1, shp.vocab), dtype=torch.int32, device="cuda")
    am_e = torch.empty(1, dtype=torch.int32, device="cuda")
    am_g = torch.empty(1, dtype=torch.int32, device="cuda")
    lg_e = torch.empty((1, shp.vocab), dtype=torch.float32, device="cuda")
    lg_g = torch.empty((1, shp.vocab), dtype=torch.float32, device="cuda")
    cur_e, cur_g = tok0.clone(), tok0.clone()
    for step in range(6):
        eager.decode_step(cur_e, am_e, lg_e)
        with torch.cuda.stream(side):
            graphed.decode_step(cur_g, am_g, lg_g)
        side.synchronize()
        torch.cuda.synchronize()
        assert np.array_equal(lg_e.cpu().numpy().view(np.uint32), lg_g.cpu().numpy().view(np.uint32)), step
        assert int(am_e.item()) == int(am_g.item())
        cur_e.copy_(am_e)
        cur_g.copy_(am_g)
        torch.cuda.synchronize()
    assert graphed.get_len(0) == 6 and graphed.status() == 0


@pytest.mark.parametrize("layers,heads", [(1, (8, 4)), (1, (8, 8)), (1, (8, 2)), (1, (16, 4)), (2, (8, 4))])
def test_decode_q8_act8_vs_oracle(layers, heads):
    """q8 x q8 products (activations quantized to int8 per 32-block on the fly) in the single-launch decode,
    against the oracle's q8 x q8 format: greedy agreement and logits cosine per step, appended K/V within
    relative L2 of the oracle's."""
    shp = replace(SMALL, fmt=synth.FMT_Q8_ACT8, n_q_heads=heads[0], n_kv_heads=heads[1], n_layers=layers)
    _say("q8 x q8", layers, heads)
    _greedy_vs_oracle(shp, seed=29, steps=12 if heads == (8, 4) else 5, kv_fill_len=20, path="mega")


@pytest.mark.parametrize("n_seq", [2, 5, 16])
def test_decode_q8_act8_batched_vs_oracle(n_seq):
    """q8 x q8 decode of several sequences: the batched products quantize each sequence's activations per
    32-block and run one int8 MFMA per block (the lm_head keeps its f16-pair operands), against the oracle's
    q8 x q8 format in its tier."""
    shp = replace(SMALL, fmt=synth.FMT_Q8_ACT8, n_seq=n_seq, max_ctx=96)
    _say("q8 x q8 batched", n_seq)
    _greedy_vs_oracle(shp, seed=31, steps=4, kv_fill_len=30,
                      seqs_checked=None if n_seq <= 5 else (0, 7, n_seq - 1))


def test_q8_act8_needs_the_single_launch_decode():
    import os
    import transformer_qwen3_block_amd as q
    W = synth.make_weights(replace(SMALL, fmt=synth.FMT_Q8_ACT8), seed=30)
    os.environ["QW3_NO_MEGA"] = "1"
    try:
        with pytest.raises(q.Qw3Error) as e:
            build_gpu_model(W)
    finally:
        os.environ.pop("QW3_NO_MEGA", None)
    assert e.value.code == 13
