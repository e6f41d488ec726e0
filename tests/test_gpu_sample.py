"""GPU parity of the deterministic sampler (qw3_sample) against the oracle's, token for token.

Both sides implement PCG32 from its published definition ("Portable WebAssembly Runtime Architecture for
TinyRustLM", "Deterministic sampling contract") and the sampling order of the same page ("Sampling order")
with "Scalar-Native Qwen3 Reference Runtime As The Numerical Authority" section 7; every floating-point step
(penalty, temperature division, max-subtracted exponentials, sums in candidate order, top-p prefix,
re-normalisation, cumulative scan) is the same IEEE f32 operation in the same order on both sides, so the drawn
token ids and the advanced generator states must be equal.  Inputs: seeded N(0, sigma) logits rows of the
Qwen3 vocabulary (151,936) and of ragged small vocabularies, seeded histories and forbidden sets.
"""
import sys

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

V = 151936


def _torch():
    import torch
    assert torch.cuda.is_available()
    return torch


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _run(rows, vocab, draws, seed, temperature, top_k, top_p, penalty, n_hist=0, forbid=(), stop=(), std=3.0,
         logits=None):
    torch = _torch()
    import transformer_qwen3_block_amd as q
    lg = logits if logits is not None else synth.logits_rows(seed, 0, rows, vocab, std)
    hist = synth.tokens(seed, 7, rows * n_hist, vocab).reshape(rows, n_hist) if n_hist else None
    fb = np.array(forbid, np.int32)
    seeds = [1000 + seed + r for r in range(rows)]
    smp = q.Sampler(rows, seeds)
    d_lg = torch.from_numpy(lg).cuda()
    d_h = torch.from_numpy(hist).cuda() if hist is not None else None
    d_f = torch.from_numpy(fb).cuda() if fb.size else None
    status = torch.empty(rows, dtype=torch.int32, device="cuda")
    done = torch.empty(rows, dtype=torch.int32, device="cuda")
    orng = [oracle.Pcg32.seeded(seeds[r], r) for r in range(rows)]
    mismatches = 0
    for d in range(draws):
        tok = smp(d_lg, temperature, top_k, top_p, penalty, d_h, d_f, stop, status=status, done=done)
        torch.cuda.synchronize()
        g_tok, g_st, g_done = tok.cpu().numpy(), status.cpu().numpy(), done.cpu().numpy()
        for r in range(rows):
            rc, o_tok, _, _ = oracle.sample(lg[r], orng[r], temperature, top_k, top_p, penalty,
                                            None if hist is None else hist[r], fb)
            assert rc == g_st[r], (d, r, rc, g_st[r])
            assert g_tok[r] == (o_tok if rc == 0 else -1), (d, r, int(g_tok[r]), o_tok)
            assert g_done[r] == (1 if rc == 0 and o_tok in stop else 0)
            mismatches += g_tok[r] != o_tok
    st = smp.rng.cpu().numpy().view(np.uint64)
    for r in range(rows):
        assert int(st[r, 0]) == orng[r].state and int(st[r, 1]) == orng[r].inc
    return lg


@pytest.mark.parametrize("rows,temperature,top_k,top_p,penalty,n_hist", [
    (1, 0.7, 50, 0.9, 1.3, 64),
    (4, 1.0, 1024, 1.0, 1.0, 0),
    (16, 0.8, 40, 0.5, 1.1, 16),
    (3, 1.5, 1, 1.0, 1.0, 0),
    (2, 0.0, 1, 1.0, 1.2, 200),      # greedy with a repetition penalty: no draw, generator untouched
    (5, 2.0, 300, 0.95, 1.0, 0),
])
def test_sampler_matches_oracle_qwen_vocab(rows, temperature, top_k, top_p, penalty, n_hist):
    _say("sample", rows, temperature, top_k, top_p, penalty, n_hist)
    _run(rows, V, draws=12, seed=51, temperature=temperature, top_k=top_k, top_p=top_p, penalty=penalty,
         n_hist=n_hist, forbid=(3, 151935, 77777), stop=(151645, 12))


@pytest.mark.parametrize("vocab", [1, 17, 1000, 4097, 262144])
def test_sampler_ragged_and_maximum_vocabularies(vocab):
    """Vocabularies that leave slices empty (1, 17), ragged slices, and the largest supported one."""
    _run(2, vocab, draws=6, seed=52, temperature=0.9, top_k=min(64, vocab), top_p=0.8, penalty=1.2,
         n_hist=8, forbid=(0,) if vocab > 1 else ())


def test_sampler_exact_ties_follow_token_ids():
    """Logits on a coarse grid (thousands of exact ties, also across slice boundaries): top-k and the
    probability order must break them by ascending id exactly as the oracle does."""
    lg = np.round(synth.logits_rows(53, 0, 4, V, 1.0) * 4) / 4
    _run(4, V, draws=8, seed=53, temperature=1.0, top_k=500, top_p=0.7, penalty=1.0, logits=lg.astype(np.float32))
    # greedy over an all-equal row: the lowest id
    flat = np.zeros((1, V), np.float32)
    _run(1, V, draws=1, seed=54, temperature=0.0, top_k=1, top_p=1.0, penalty=1.0, logits=flat)


def test_sampler_non_finite_rows():
    """NaN logits are never drawn; a +inf logit or a row without a finite logit reports NumericalFailure with
    token -1 (and leaves that row's generator untouched, as the oracle does)."""
    lg = synth.logits_rows(55, 0, 4, 5000, 2.0)
    lg[0, ::3] = np.nan
    lg[1, 17] = np.inf
    lg[2, :] = -np.inf
    lg[3, :] = np.nan
    _run(4, 5000, draws=3, seed=55, temperature=0.9, top_k=100, top_p=0.9, penalty=1.0, logits=lg)


def test_sampler_on_decode_logits():
    """Sampling straight from a decode step's logits buffer ([n_seq][vocab]) in a generation loop: each
    drawn token is fed to the next step, and the oracle's sampler, given the same logits, draws the same."""
    torch = _torch()
    from dataclasses import replace
    from parity import build_gpu_model
    import transformer_qwen3_block_amd as q
    shp = replace(synth.QWEN3_06B, fmt=synth.FMT_Q8, vocab=4000, n_layers=2, n_q_heads=8, n_kv_heads=4,
                  inter=1024, max_ctx=64, n_seq=3, max_prefill=8)
    m = build_gpu_model(synth.make_weights(shp, seed=56))
    smp = q.Sampler(shp.n_seq, [5, 6, 7])
    orng = [oracle.Pcg32.seeded(s, r) for r, s in enumerate([5, 6, 7])]
    cur = torch.from_numpy(synth.tokens(56, 1, shp.n_seq, shp.vocab)).cuda()
    am = torch.empty(shp.n_seq, dtype=torch.int32, device="cuda")
    lg = torch.empty((shp.n_seq, shp.vocab), dtype=torch.float32, device="cuda")
    hist = []
    for step in range(8):
        m.decode_step(cur, am, lg)
        hist.append(cur.clone())
        h = torch.stack(hist, 1).contiguous()
        tok = smp(lg, temperature=0.8, top_k=40, top_p=0.9, penalty=1.1, history=h)
        torch.cuda.synchronize()
        g = lg.cpu().numpy()
        hh = h.cpu().numpy()
        for r in range(shp.n_seq):
            rc, o_tok, _, _ = oracle.sample(g[r], orng[r], 0.8, 40, 0.9, 1.1, hh[r])
            assert rc == 0 and int(tok[r].item()) == o_tok, (step, r)
        cur = tok
    assert m.status() == 0
