"""Full-size workloads on the GPU, in the launch configuration bench.py times.

Each is compared with the oracle on outputs it can compute one by one (sampled sequences and steps), or
through a property that holds at any size (tiled prefill vs the GPU's own token-by-token path).
Inputs follow the workload recipes (synth.WORKLOADS): Q8 codes uniform in [-127,127], scales U(1e-3,1e-2),
bf16 weights N(0,0.02), norms 1+N(0,0.1), KV fills bf16 N(0,1).
"""
import sys
import time
from dataclasses import replace

import numpy as np
import pytest

import oracle
import synth
from parity import Margins, argmax_ok, assert_close, build_gpu_model, forced_step

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    assert torch.cuda.is_available()
    return torch


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _fill_kv(m, orc_by_seq, seed, shp, seqs, n_pos):
    torch = _torch()
    for s in seqs:
        for l in range(shp.n_layers):
            k, v = synth.kv_fill(seed, s, l, shp.n_kv_heads, n_pos, shp.head_dim)
            m.kv_write(s, l, 0, torch.from_numpy(k.view(np.int16)).cuda(), torch.from_numpy(v.view(np.int16)).cuda())
            if s in orc_by_seq:
                orc_by_seq[s].kv_write(0, l, 0, k, v)
        m.set_len(s, n_pos)
        if s in orc_by_seq:
            orc_by_seq[s].set_len(0, n_pos)
    torch.cuda.synchronize()


@pytest.mark.timeout(300)
def test_q8_0_blocks_decode_context_2048_full():
    """The same 28-layer decode at KV context 2048 with the weights given as the pages' Q8_0 blocks (f16
    scales, 34 bytes per 32 inputs), against the oracle reading those blocks: 8 greedy steps."""
    torch = _torch()
    wl = synth.Q8_DECODE
    shp = replace(wl.shape, fmt=synth.FMT_Q8_0)
    W = synth.make_weights(shp, seed=wl.seed)
    m = build_gpu_model(W)
    orc = oracle.Model(W, n_seq=1)
    _fill_kv(m, {0: orc}, wl.seed, shp, [0], wl.kv_prefill)
    cur = torch.tensor(synth.tokens(wl.seed, 1, 1, shp.vocab), dtype=torch.int32, device="cuda")
    am = torch.empty(1, dtype=torch.int32, device="cuda")
    lg = torch.empty((1, shp.vocab), dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    worst = Margins("28-layer Q8_0-block decode, KV context 2048..2055")
    kv = {}
    for step in range(8):
        with torch.cuda.stream(side):
            m.decode_step(cur, am, lg)
        side.synchronize()
        rc, _, o_lg, _ = forced_step(m, orc, 0, int(cur.item()), shp.n_layers, stats=kv)
        assert rc == 0
        g = lg.cpu().numpy()[0]
        worst.add(assert_close(g, o_lg, f"step {step}"))
        assert argmax_ok(int(am.item()), o_lg, g)
        cur = am.clone()
    worst.report(kv)
    assert m.status() == 0


@pytest.mark.timeout(300)
def test_q8_act8_decode_context_2048_full():
    """The 28-layer decode at KV context 2048 with q8 x q8 layer products (int8 activations), against the
    oracle's q8 x q8 format in the deep tier: greedy agreement and logits cosine >= 0.99 per step, 8 steps."""
    from parity import ACT8_COS, cosine, forced_step_act8
    torch = _torch()
    wl = synth.Q8_DECODE
    shp = replace(wl.shape, fmt=synth.FMT_Q8_ACT8)
    W = synth.make_weights(shp, seed=wl.seed)
    m = build_gpu_model(W)
    orc = oracle.Model(W, n_seq=1)
    _fill_kv(m, {0: orc}, wl.seed, shp, [0], wl.kv_prefill)
    cur = torch.tensor(synth.tokens(wl.seed, 1, 1, shp.vocab), dtype=torch.int32, device="cuda")
    am = torch.empty(1, dtype=torch.int32, device="cuda")
    lg = torch.empty((1, shp.vocab), dtype=torch.float32, device="cuda")
    worst_cos, st = 1.0, {}
    for step in range(8):
        m.decode_step(cur, am, lg)
        torch.cuda.synchronize()
        rc, _, o_lg, _ = forced_step_act8(m, orc, 0, int(cur.item()), shp.n_layers, stats=st)
        assert rc == 0
        g = lg.cpu().numpy()[0]
        c = cosine(g, o_lg)
        worst_cos = min(worst_cos, c)
        assert c >= ACT8_COS and argmax_ok(int(am.item()), o_lg, g), (step, c)
        cur = am.clone()
    _say(f"MARGIN 28-layer q8 x q8 decode: worst logits cosine {worst_cos:.6f} (bound {ACT8_COS}), worst appended "
         f"K/V rel-L2 {st.get('kv_rel', 0):.3e}")
    assert m.status() == 0


@pytest.mark.timeout(600)
def test_q8_decode_context_2048_full():
    """28-layer Q8 B=1 decode over a 2048-position KV cache: 64 greedy steps, every step checked against the
    oracle (teacher forced), in the graph-replayed side-stream launch of bench.py."""
    torch = _torch()
    wl = synth.Q8_DECODE
    shp = wl.shape
    _say("Q8 decode full size", shp)
    W = synth.make_weights(shp, seed=wl.seed)
    m = build_gpu_model(W)
    orc = oracle.Model(W, n_seq=1)
    _fill_kv(m, {0: orc}, wl.seed, shp, [0], wl.kv_prefill)
    cur = torch.tensor(synth.tokens(wl.seed, 1, 1, shp.vocab), dtype=torch.int32, device="cuda")
    am = torch.empty(1, dtype=torch.int32, device="cuda")
    lg = torch.empty((1, shp.vocab), dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    steps = 64
    worst = Margins("28-layer Q8 decode, KV context 2048..2111")
    kv = {}
    for step in range(steps):
        with torch.cuda.stream(side):   # the graph-replayed launch configuration of bench.py
            m.decode_step(cur, am, lg)
        side.synchronize()
        rc, _, o_lg, _ = forced_step(m, orc, 0, int(cur.item()), shp.n_layers, stats=kv)
        assert rc == 0
        g = lg.cpu().numpy()[0]
        mab, r = assert_close(g, o_lg, f"step {step}")
        worst.add((mab, r))
        if step % 16 == 0:
            _say(f"  step {step}: max-abs {mab:.3e} rel-L2 {r:.3e} (logit rms {np.sqrt(np.mean(o_lg ** 2)):.2f})")
        assert argmax_ok(int(am.item()), o_lg, g)
        cur = am.clone()
    worst.report(kv)
    assert m.get_len(0) == wl.kv_prefill + steps and m.status() == 0


@pytest.mark.parametrize("fmt", [synth.FMT_Q8, synth.FMT_Q8_ACT8])
def test_batched_16_sequences_context_8192_full(fmt):
    """16 sequences x 8192-position caches, Q8 (and the q8 x q8 format: int8 activations on int8 MFMA), one
    greedy step per sequence per iteration; sequences 0 and 15 are replayed through the oracle (sequences are
    independent).  The q8 x q8 format is compared in its tier: greedy agreement and logits cosine."""
    from parity import ACT8_COS, cosine, forced_step_act8
    torch = _torch()
    wl = synth.Q8_BATCHED
    shp = replace(wl.shape, fmt=fmt)
    act8 = fmt == synth.FMT_Q8_ACT8
    _say("batched full size", shp)
    t0 = time.time()
    W = synth.make_weights(shp, seed=wl.seed)
    m = build_gpu_model(W)
    check = (0, shp.n_seq - 1)
    orcs = {s: oracle.Model(W, n_seq=1) for s in check}
    _fill_kv(m, orcs, wl.seed, shp, range(shp.n_seq), wl.kv_prefill)
    _say(f"  filled in {time.time() - t0:.1f}s")
    cur = torch.from_numpy(synth.tokens(wl.seed, 1, shp.n_seq, shp.vocab)).cuda()
    am = torch.empty(shp.n_seq, dtype=torch.int32, device="cuda")
    lg = torch.empty((shp.n_seq, shp.vocab), dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    worst = Margins(f"16 x 8192 batched {'q8 x q8' if act8 else 'Q8'}, sequences 0 and 15")
    kv = {}
    worst_cos = 1.0
    for it in range(2):
        with torch.cuda.stream(side):
            m.decode_step(cur, am, lg)
        side.synchronize()
        g_all = lg.cpu().numpy()
        for s in check:
            if act8:
                rc, _, o_lg, _ = forced_step_act8(m, orcs[s], s, int(cur[s].item()), shp.n_layers, orc_seq=0,
                                                  stats=kv)
                assert rc == 0
                cs = cosine(g_all[s], o_lg)
                worst_cos = min(worst_cos, cs)
                assert cs >= ACT8_COS, (it, s, cs)
            else:
                rc, _, o_lg, _ = forced_step(m, orcs[s], s, int(cur[s].item()), shp.n_layers, orc_seq=0, stats=kv)
                assert rc == 0
                mab, r = assert_close(g_all[s], o_lg, f"iteration {it} seq {s}")
                worst.add((mab, r))
            assert argmax_ok(int(am[s].item()), o_lg, g_all[s])
        cur = am.clone()
    if act8:
        _say(f"MARGIN 16 x 8192 batched q8 x q8: worst logits cosine {worst_cos:.6f} (bound {ACT8_COS}), worst "
             f"appended K/V rel-L2 {kv.get('kv_rel', 0):.3e}")
    else:
        worst.report(kv)
    assert m.status() == 0
    for s in range(shp.n_seq):
        assert m.get_len(s) == wl.kv_prefill + 2


def test_prefill_2048_full_tiled_vs_token_path():
    """28-layer bf16 prefill of 2048 tokens (one MFMA tile) against prefill(2047) + decode(1) on the GPU."""
    torch = _torch()
    wl = synth.BF16_PREFILL
    shp = replace(wl.shape, max_ctx=2048)
    W = synth.make_weights(shp, seed=wl.seed)
    a = build_gpu_model(W)
    toks = torch.from_numpy(synth.tokens(wl.seed, 0, wl.prefill, shp.vocab)).cuda()
    la = torch.empty(shp.vocab, dtype=torch.float32, device="cuda")
    am = torch.empty(1, dtype=torch.int32, device="cuda")
    a.prefill(toks, 0, la, am)
    torch.cuda.synchronize()
    g_a = la.cpu().numpy()
    am_a = int(am.item())
    a.reset_kv(0)
    a.prefill(toks[:-1].contiguous(), 0, None, am)
    lb = torch.empty((1, shp.vocab), dtype=torch.float32, device="cuda")
    a.decode_step(toks[-1:].contiguous(), am, lb)
    torch.cuda.synchronize()
    mab, r = assert_close(g_a, lb.cpu().numpy()[0], "prefill(2048) vs prefill(2047)+decode")
    _say(f"  max-abs {mab:.3e} rel-L2 {r:.3e}")
    assert argmax_ok(am_a, lb.cpu().numpy()[0], g_a)
    assert a.status() == 0


@pytest.mark.timeout(900)
@pytest.mark.parametrize("n_layers", [2, 28])
def test_prefill_2048_vs_oracle(n_layers):
    """The 2048-token prompt through the tiled f16-operand MFMA prefill, last-position logits against the
    oracle's token-by-token prefill: at 2 layers, and at the workload's full 28 layers (the oracle takes
    about a minute and a half on the host threads)."""
    torch = _torch()
    wl = synth.BF16_PREFILL
    shp = replace(wl.shape, n_layers=n_layers)
    W = synth.make_weights(shp, seed=wl.seed)
    m = build_gpu_model(W)
    toks = synth.tokens(wl.seed, 0, wl.prefill, shp.vocab)
    lg = torch.empty(shp.vocab, dtype=torch.float32, device="cuda")
    am = torch.empty(1, dtype=torch.int32, device="cuda")
    m.prefill(torch.from_numpy(toks).cuda(), 0, lg, am)
    torch.cuda.synchronize()
    t0 = time.time()
    rc, _, o_lg = oracle.Model(W).prefill(toks)
    _say(f"  oracle prefill 2048 x {n_layers} layers: {time.time() - t0:.1f}s")
    assert rc == 0
    mab, r = assert_close(lg.cpu().numpy(), o_lg, f"{n_layers}-layer prefill 2048")
    w = Margins(f"prefill 2048, {n_layers} layers, last-position logits")
    w.add((mab, r))
    w.report()
    assert argmax_ok(int(am.item()), o_lg, lg.cpu().numpy())
