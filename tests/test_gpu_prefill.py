"""GPU parity of the tiled bf16 MFMA prefill against the oracle's token-by-token prefill (through the C ABI).

Prompt lengths are ragged (not multiples of the 16/32/64/128 tiles) and longer than one prefill tile, so
the GEMM row guards, the causal diagonal tiles and the tile-by-tile KV publication are all exercised.  The
tiled prefill is also compared with the GPU's own token-by-token path (prefill T-1, then decode 1), which
shares no kernel with it.
"""
import sys
from dataclasses import replace

import numpy as np
import pytest

import oracle
import synth
from parity import Margins, argmax_ok, assert_close, build_gpu_model, forced_step, rel_l2, sync_prefilled_kv

pytestmark = pytest.mark.gpu

SMALL = replace(synth.QWEN3_06B, vocab=1000, n_layers=2, n_q_heads=8, n_kv_heads=4, inter=1024, max_ctx=320,
                max_prefill=256)


def _torch():
    import torch
    assert torch.cuda.is_available()
    return torch


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _prefill_vs_oracle(shp, seed, T, decode_steps=0):
    torch = _torch()
    _say("prefill", T, shp)
    W = synth.make_weights(shp, seed=seed)
    m = build_gpu_model(W)
    orc = oracle.Model(W)
    toks = synth.tokens(seed, 0, T, shp.vocab)
    logits = torch.empty(shp.vocab, dtype=torch.float32, device="cuda")
    am = torch.empty(1, dtype=torch.int32, device="cuda")
    m.prefill(torch.from_numpy(toks).cuda(), 0, logits, am)
    torch.cuda.synchronize()
    rc, o_am, o_logits = orc.prefill(toks)
    assert rc == 0
    g = logits.cpu().numpy()
    mab, r = assert_close(g, o_logits, f"prefill T={T}")
    first = Margins(f"prefill T={T} layers={shp.n_layers} last-position logits")
    first.add((mab, r))
    first.report()
    assert argmax_ok(int(am.item()), o_logits, g)
    assert m.get_len(0) == T and orc.get_len(0) == T
    # decode on top of the prefilled cache, teacher forced: first the whole prompt cache, then each step's append
    if decode_steps:
        _say(f"  prompt cache rel-L2 against the oracle's: {sync_prefilled_kv(m, orc, 0, T, shp.n_layers):.3e}")
    cur = am.clone().reshape(1)
    lg = torch.empty((1, shp.vocab), dtype=torch.float32, device="cuda")
    worst = Margins(f"decode after prefill {T}, layers={shp.n_layers}")
    kv = {}
    ids = []
    for step in range(decode_steps):
        m.decode_step(cur, am, lg)
        torch.cuda.synchronize()
        rc, _, o_lg, _ = forced_step(m, orc, 0, int(cur.item()), shp.n_layers, stats=kv)
        assert rc == 0
        worst.add(assert_close(lg.cpu().numpy()[0], o_lg, f"decode {step} after prefill {T}"))
        assert argmax_ok(int(am.item()), o_lg, lg.cpu().numpy()[0])
        ids.append(int(am.item()))
        cur = am.clone()
    if decode_steps:
        worst.report(kv)
        _say("  greedy ids:", ids)
    assert m.status() == 0
    return m, W


@pytest.mark.parametrize("T", [1, 37, 200])
def test_prefill_small_vs_oracle(T):
    _prefill_vs_oracle(SMALL, seed=31, T=T, decode_steps=3)


def test_prefill_several_tiles():
    """A prompt longer than one prefill tile runs tile by tile; later tiles attend to earlier ones."""
    _prefill_vs_oracle(replace(SMALL, max_prefill=48), seed=32, T=130, decode_steps=2)


def test_prefill_single_token_tiles_bf16():
    """A bf16 model configured with one-token prefill tiles has no MFMA prefill: its prompt runs token by token
    through the decode path (f32 activations), and the logits and cache still match the oracle."""
    _prefill_vs_oracle(replace(SMALL, max_prefill=1), seed=37, T=12, decode_steps=2)


@pytest.mark.parametrize("chunk,T", [(600, 1250), (128, 300), (100, 290), (256, 256), (512, 512), (520, 513)])
def test_prefill_chunks_every_projection_path(chunk, T):
    """Chunked prefill through every projection path.  Chunks of more than 512 tokens (600, 513) take the tiled
    products with the fused Q/K/V epilogue, which writes the attention's f16 K/V shadow when the chunk starts on
    a 64-position boundary (0) and leaves it to the conversion kernel when not (600); chunks of 512 tokens or
    fewer (128, 100, 50, 44, 90, and exactly 256 and 512) split K over more workgroups, with the QK-Norm kernel
    adding the projection's K ranges and the residual products' reductions normalising for the next product.
    The attention runs each query block's keys in one workgroup while the causal range stays within 256 keys
    (first chunks of 100, 128 and 256 tokens, and the second of 100 or 128 at a nonzero start) and splits them
    between two workgroups past it."""
    _prefill_vs_oracle(replace(SMALL, max_prefill=chunk, max_ctx=1280), seed=36, T=T, decode_steps=2)


@pytest.mark.parametrize("heads", [(8, 8), (8, 2)])
def test_prefill_gqa_group_sizes(heads):
    shp = replace(SMALL, n_q_heads=heads[0], n_kv_heads=heads[1], n_layers=1)
    _prefill_vs_oracle(shp, seed=33, T=70)


def test_prefill_kv_cache_close_to_oracle():
    """Keys/values the prefill appended (bf16 MFMA projections) match the oracle's cache per head."""
    torch = _torch()
    m, W = _prefill_vs_oracle(SMALL, seed=34, T=45)
    orc = oracle.Model(W)
    orc.prefill(synth.tokens(34, 0, 45, SMALL.vocab))
    for layer in range(SMALL.n_layers):
        k, v = m.kv_read(0, layer, 0, 45)
        _, ok, ov = orc.kv_read(0, layer, 0, 45)
        kg = synth.bf16_to_f32(k.cpu().numpy().view(np.uint16))
        vg = synth.bf16_to_f32(v.cpu().numpy().view(np.uint16))
        assert rel_l2(kg, synth.bf16_to_f32(ok)) < 1e-2
        assert rel_l2(vg, synth.bf16_to_f32(ov)) < 1e-2


def test_tiled_prefill_equals_token_by_token_gpu():
    """prefill(T) against prefill(T-1) + decode(1): two independent GPU paths, same logits."""
    torch = _torch()
    W = synth.make_weights(SMALL, seed=35)
    a = build_gpu_model(W)
    b = build_gpu_model(W)
    toks = torch.from_numpy(synth.tokens(35, 0, 90, SMALL.vocab)).cuda()
    la = torch.empty(SMALL.vocab, dtype=torch.float32, device="cuda")
    am = torch.empty(1, dtype=torch.int32, device="cuda")
    a.prefill(toks, 0, la, am)
    b.prefill(toks[:89].contiguous(), 0, None, am)
    lb = torch.empty((1, SMALL.vocab), dtype=torch.float32, device="cuda")
    b.decode_step(toks[89:90].contiguous(), am, lb)
    torch.cuda.synchronize()
    assert_close(la.cpu().numpy(), lb.cpu().numpy()[0], "prefill(90) vs prefill(89)+decode")


def test_single_block_workload():
    """Single Qwen3-0.6B block, bf16, fp32 hidden inputs N(0,1): prefill 16 positions (MFMA path), then
    16 decode positions; all 32 output hidden states against the oracle."""
    torch = _torch()
    wl = synth.SINGLE_BLOCK
    shp = wl.shape
    W = synth.make_weights(shp, seed=wl.seed)
    m = build_gpu_model(W)
    orc = oracle.Model(W)
    hin = synth.hidden_inputs(wl.seed, 0, wl.prefill + wl.hidden_decode, shp.hidden)
    out = torch.empty((wl.prefill, shp.hidden), dtype=torch.float32, device="cuda")
    m.block_forward(torch.from_numpy(hin[:wl.prefill]).cuda(), out)
    torch.cuda.synchronize()
    g = out.cpu().numpy()
    worst = Margins("single block, 32 output hidden states")
    for t in range(wl.prefill):
        rc, _, _, ref = orc.step(0, hidden_in=hin[t], want_hidden=True)
        assert rc == 0
        worst.add(assert_close(g[t], ref, f"prefill position {t}"))
    one = torch.empty((1, shp.hidden), dtype=torch.float32, device="cuda")
    for t in range(wl.prefill, wl.prefill + wl.hidden_decode):
        m.block_forward(torch.from_numpy(hin[t:t + 1]).cuda(), one)
        torch.cuda.synchronize()
        rc, _, _, ref = orc.step(0, hidden_in=hin[t], want_hidden=True)
        assert rc == 0
        worst.add(assert_close(one.cpu().numpy()[0], ref, f"decode position {t}"))
    worst.report()
    assert m.get_len(0) == 32


@pytest.mark.timeout(600)
def test_full_size_prefill_128_then_decode():
    """28-layer Qwen3-0.6B shape, bf16, 128-token prefill then all 256 greedy decode steps of the workload
    (teacher forced), contexts 129..384."""
    wl = synth.BF16_DECODE
    _prefill_vs_oracle(wl.shape, seed=wl.seed, T=wl.prefill, decode_steps=wl.decode)
