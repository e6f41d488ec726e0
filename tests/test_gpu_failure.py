"""GPU checks of the greedy choice's edge cases and of the failure contract, through the C ABI.

- Exact ties: the greedy choice takes the lowest token id among equal maxima ("Portable WebAssembly Runtime
  Architecture for TinyRustLM", "Sampling order").  Two vocabulary rows are made byte-identical, so their
  tied logits are bit-identical on both sides; the oracle picks the lower id as well.
- NaN/Inf: a non-finite logit aborts the generation with a typed error and never a repaired value
  ("Scalar-Native Qwen3 Reference Runtime As The Numerical Authority", section 4 "NaN/Inf Rejection"); the
  failing step commits nothing, steps completed before it stand (section 8), and the handle refuses work
  until reset.  NaN enters as ordinary data (a cached value or a norm weight): no kernel faults.
- The launch configuration the benchmark times (tokens aliasing the previous argmax, no logits buffer,
  graph replay on a side stream) gives the same greedy trajectory as a run with logits.
"""
import sys
from dataclasses import replace

import numpy as np
import pytest

import oracle
import synth
from parity import build_gpu_model

pytestmark = pytest.mark.gpu

SMALL = replace(synth.QWEN3_06B, vocab=1000, n_layers=2, n_q_heads=8, n_kv_heads=4, inter=1024, max_ctx=64,
                max_prefill=32)
NUMERICAL_FAILURE = 18


def _torch():
    import torch
    assert torch.cuda.is_available()
    return torch


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _build(W, path):
    import os
    if path == "kernels":
        os.environ["QW3_NO_MEGA"] = "1"
    try:
        return build_gpu_model(W)
    finally:
        os.environ.pop("QW3_NO_MEGA", None)


def _copy_row(m, src, dst):
    if m.is_q8:
        m.codes[dst] = m.codes[src]
        m.scales[dst] = m.scales[src]
    else:
        m.bf16[dst] = m.bf16[src]


@pytest.mark.parametrize("path", ["mega", "kernels"])
@pytest.mark.parametrize("fmt", [synth.FMT_BF16, synth.FMT_Q8])
@pytest.mark.parametrize("twin_above", [True, False])
def test_exact_argmax_tie_takes_lowest_id(fmt, path, twin_above):
    """The oracle's first greedy choice a gets a byte-identical twin row b (b > a or b < a); with tied
    embeddings the two logits are equal bit for bit, and both sides must return min(a, b)."""
    torch = _torch()
    shp = replace(SMALL, fmt=fmt)
    W = synth.make_weights(shp, seed=41)
    tok = int(synth.tokens(41, 1, 1, shp.vocab)[0])
    _, a, lg, _ = oracle.Model(W).step(0, tok)
    b = a + 37 if twin_above else a - 37
    if not 0 <= b < shp.vocab or tok in (a, b):
        b = a + 1 if twin_above else a - 1
    assert 0 <= b < shp.vocab and tok not in (a, b)
    _copy_row(W.embed, a, b)
    _say("tie", fmt, path, "rows", a, b)
    rc, o_am, o_lg, _ = oracle.Model(W).step(0, tok)
    assert rc == 0 and o_lg[a] == o_lg[b] and o_am == min(a, b)
    m = _build(W, path)
    am = torch.empty(1, dtype=torch.int32, device="cuda")
    lgt = torch.empty((1, shp.vocab), dtype=torch.float32, device="cuda")
    m.decode_step(torch.tensor([tok], dtype=torch.int32, device="cuda"), am, lgt)
    torch.cuda.synchronize()
    g = lgt.cpu().numpy()[0]
    assert g[a].view(np.uint32) == g[b].view(np.uint32)
    assert g[a] == g.max(), "the tied rows carry the maximum"
    assert int(am.item()) == min(a, b)
    assert m.status() == 0


def test_exact_argmax_tie_batched_sequences():
    """The batched Q8 logits (MFMA) pick the lowest id of a bit-identical tie in every sequence."""
    torch = _torch()
    shp = replace(SMALL, fmt=synth.FMT_Q8, n_seq=4)
    W = synth.make_weights(shp, seed=42)
    toks = synth.tokens(42, 1, shp.n_seq, shp.vocab)
    orc = oracle.Model(W, n_seq=1)
    _, a, _, _ = orc.step(0, int(toks[0]))
    b = a - 1 if a > 0 else a + 1
    _copy_row(W.embed, a, b)
    m = build_gpu_model(W)
    am = torch.empty(shp.n_seq, dtype=torch.int32, device="cuda")
    lgt = torch.empty((shp.n_seq, shp.vocab), dtype=torch.float32, device="cuda")
    m.decode_step(torch.from_numpy(toks).cuda(), am, lgt)
    torch.cuda.synchronize()
    g = lgt.cpu().numpy()
    assert g[0, a].view(np.uint32) == g[0, b].view(np.uint32)
    if g[0, a] == g[0].max():
        assert int(am[0].item()) == min(a, b)
    for s in range(shp.n_seq):   # every sequence: the reported id is the lowest among its maxima
        assert int(am[s].item()) == int(np.flatnonzero(g[s] == g[s].max())[0])


@pytest.mark.parametrize("path", ["mega", "kernels"])
def test_nan_in_cache_latches_failure_and_commits_nothing(path):
    """Two good steps, then a NaN planted in a committed cache position: the next step's logits are NaN, the
    step commits nothing (length stays at the last good step), the poll reports NumericalFailure, every later
    call is refused, and reset_kv brings the handle back."""
    torch = _torch()
    import transformer_qwen3_block_amd as q
    shp = replace(SMALL, fmt=synth.FMT_Q8)
    W = synth.make_weights(shp, seed=43)
    m = _build(W, path)
    for l in range(shp.n_layers):
        k, v = synth.kv_fill(43, 0, l, shp.n_kv_heads, 10, shp.head_dim)
        m.kv_write(0, l, 0, torch.from_numpy(k.view(np.int16)).cuda(), torch.from_numpy(v.view(np.int16)).cuda())
    m.set_len(0, 10)
    cur = torch.tensor(synth.tokens(43, 1, 1, shp.vocab), dtype=torch.int32, device="cuda")
    am = torch.empty(1, dtype=torch.int32, device="cuda")
    lgt = torch.empty((1, shp.vocab), dtype=torch.float32, device="cuda")
    good = []
    for _ in range(2):
        m.decode_step(cur, am, lgt)
        torch.cuda.synchronize()
        good.append(int(am.item()))
        cur = am.clone()
    assert m.status() == 0 and m.get_len(0) == 12
    # a NaN value in KV head 0, position 3 of layer 1 (bf16 quiet NaN); every query head of that KV head
    # attends to it
    k, v = m.kv_read(0, 1, 3, 1)
    vb = v.cpu().numpy().view(np.uint16).copy()
    vb[0, 0, 5] = 0x7FC0
    m.kv_write(0, 1, 3, k, torch.from_numpy(vb.view(np.int16)).cuda())
    m.decode_step(cur, am, lgt)
    torch.cuda.synchronize()
    assert not np.all(np.isfinite(lgt.cpu().numpy()))
    assert m.status() == NUMERICAL_FAILURE
    assert m.get_len(0) == 12, "the failing step committed nothing"
    with pytest.raises(q.Qw3Error) as e:
        m.decode_step(cur, am, lgt)
    assert e.value.code == NUMERICAL_FAILURE and m.get_len(0) == 12
    with pytest.raises(q.Qw3Error) as e:
        m.prefill(cur, 0, None, am)
    assert e.value.code == NUMERICAL_FAILURE
    # the completed steps' argmax matched a fresh run's (they stay valid)
    m.reset_kv(0)
    assert m.get_len(0) == 0 and m.status() == 0
    m.decode_step(cur, am, lgt)
    torch.cuda.synchronize()
    assert np.all(np.isfinite(lgt.cpu().numpy())) and m.status() == 0 and m.get_len(0) == 1
    _say("good steps before the failure:", good)


def test_nan_norm_weight_fails_first_step_bf16_prefill_and_decode():
    """A NaN final-norm weight makes every logit NaN: the tiled prefill and the decode step both latch
    NumericalFailure and commit nothing."""
    torch = _torch()
    shp = replace(SMALL, max_ctx=96, max_prefill=48)
    W = synth.make_weights(shp, seed=44)
    W.final_norm = W.final_norm.copy()
    W.final_norm[17] = 0x7FC0
    m = build_gpu_model(W)
    toks = torch.from_numpy(synth.tokens(44, 0, 70, shp.vocab)).cuda()   # two prefill tiles
    am = torch.empty(1, dtype=torch.int32, device="cuda")
    lg = torch.empty(shp.vocab, dtype=torch.float32, device="cuda")
    m.prefill(toks, 0, lg, am)
    torch.cuda.synchronize()
    assert np.all(np.isnan(lg.cpu().numpy()))
    assert m.status() == NUMERICAL_FAILURE
    # the first tile's commit happened before the failure was found (stream order), the last tile's did not
    assert m.get_len(0) == 48
    m.reset_kv(0)
    m.decode_step(toks[:1].contiguous(), am)
    assert m.status() == NUMERICAL_FAILURE and m.get_len(0) == 0


def test_invalid_token_is_reported_and_stops_commits():
    """A token id outside [0, vocab) reaching the device is reported (InvalidArgument) and nothing commits."""
    torch = _torch()
    m = build_gpu_model(synth.make_weights(replace(SMALL, fmt=synth.FMT_Q8), seed=45))
    am = torch.empty(1, dtype=torch.int32, device="cuda")
    m.decode_step(torch.tensor([SMALL.vocab + 5], dtype=torch.int32, device="cuda"), am)
    assert m.status() == 1 and m.get_len(0) == 0
    m.reset_kv(-1)
    m.decode_step(torch.tensor([3], dtype=torch.int32, device="cuda"), am)
    assert m.status() == 0 and m.get_len(0) == 1


def test_timed_configuration_matches_logits_run_full_size():
    """The benchmark's launch configuration -- 28-layer Q8 at KV context 2048, tokens aliasing the argmax
    buffer, no logits buffer, graph replay on a side stream -- gives the same greedy trajectory as steps with
    separate token and logits buffers (which the oracle parity tests compare)."""
    torch = _torch()
    wl = synth.Q8_DECODE
    shp = wl.shape
    W = synth.make_weights(shp, seed=wl.seed)
    m = build_gpu_model(W)
    for l in range(shp.n_layers):
        k, v = synth.kv_fill(wl.seed, 0, l, shp.n_kv_heads, wl.kv_prefill, shp.head_dim)
        m.kv_write(0, l, 0, torch.from_numpy(k.view(np.int16)).cuda(), torch.from_numpy(v.view(np.int16)).cuda())
    m.set_len(0, wl.kv_prefill)
    start = synth.tokens(wl.seed, 1, 1, shp.vocab)
    side = torch.cuda.Stream()
    steps = 24
    am = torch.tensor(start, dtype=torch.int32, device="cuda")
    timed = []
    for _ in range(steps):
        with torch.cuda.stream(side):
            m.decode_step(am, am)            # tokens alias argmax, logits NULL
        side.synchronize()
        timed.append(int(am.item()))
    assert m.status() == 0 and m.get_len(0) == wl.kv_prefill + steps
    m.set_len(0, wl.kv_prefill)
    cur = torch.tensor(start, dtype=torch.int32, device="cuda")
    out = torch.empty(1, dtype=torch.int32, device="cuda")
    lg = torch.empty((1, shp.vocab), dtype=torch.float32, device="cuda")
    ref = []
    for _ in range(steps):
        m.decode_step(cur, out, lg)
        torch.cuda.synchronize()
        ref.append(int(out.item()))
        cur.copy_(out)
    _say("timed trajectory", timed)
    assert timed == ref
