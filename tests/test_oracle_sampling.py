"""Pins of the oracle's deterministic sampler against what the pages and the mathematics fix (CPU only).

Sources: "Scalar-Native Qwen3 Reference Runtime As The Numerical Authority" section 7 (stable softmax,
repetition penalty, tie-breaking sort, top-k, top-p, selection) and section 9 ("Repetition Penalty
Inversion"); "Portable WebAssembly Runtime Architecture for TinyRustLM", "Deterministic sampling contract"
(PCG32 transition, output, seeding, 24-bit uniform) and "Sampling order".
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_pcg32_known_answer_words():
    kat = json.load(open(os.path.join(GOLDEN, "pcg32_kat.json")))
    r = oracle.Pcg32.seeded(kat["seed"], kat["stream"])
    assert [r.next() for _ in range(len(kat["words"]))] == [int(w, 16) for w in kat["words"]]


def test_uniform_is_the_exact_high_24_bits():
    assert oracle.pcg32_uniform(0) == 0.0
    assert oracle.pcg32_uniform(0xFFFFFFFF) == (2 ** 24 - 1) / 2 ** 24    # < 1, exact
    assert oracle.pcg32_uniform(0x80000000) == 0.5
    assert oracle.pcg32_uniform(0x000000FF) == 0.0                       # low byte ignored


def test_repetition_penalty_inversion():
    """The section 9 vector: a positive repeated logit shrinks, a negative one grows in magnitude; zero,
    unrepeated and out-of-range history entries are untouched, and a repeated id is penalised once."""
    rc, z = oracle.sample_prepare([2.0, -2.0, 0.0, 3.0, -1.0], penalty=1.5, history=[0, 1, 2, 1, 0, 99, -1])
    assert rc == 0
    assert z[0] == np.float32(2.0) / np.float32(1.5) and z[1] == -3.0
    assert z[2] == 0.0 and z[3] == 3.0 and z[4] == -1.0


def test_prepare_masks_nan_and_negative_zero():
    rc, z = oracle.sample_prepare([np.nan, -0.0, 1.0, 5.0], forbid=[3])
    assert rc == 0
    assert z[0] == -np.inf and z[3] == -np.inf
    assert z[1] == 0.0 and not np.signbit(z[1])
    rc, _ = oracle.sample_prepare([1.0, np.inf])
    assert rc == oracle.ORC_NUMERICAL_FAILURE


def test_greedy_lowest_id_on_ties_and_no_draw():
    r = oracle.Pcg32.seeded(1, 2)
    before = (r.state, r.inc)
    rc, tok, _, _ = oracle.sample([1.0, 3.0, -2.0, 3.0], r, temperature=0.0)
    assert rc == 0 and tok == 1
    assert (r.state, r.inc) == before


def test_top_k_one_is_greedy():
    rng = np.random.default_rng(0)
    lg = rng.standard_normal(200).astype(np.float32)
    r = oracle.Pcg32.seeded(3, 0)
    for _ in range(20):
        rc, tok, ids, probs = oracle.sample(lg, r, temperature=0.7, top_k=1)
        assert rc == 0 and tok == int(np.argmax(lg)) and list(ids) == [tok] and probs[0] == 1.0


def test_candidates_follow_value_then_id_order():
    lg = np.array([1.0, 2.0, 2.0, 0.5, 2.0, -1.0], np.float32)
    rc, _, ids, probs = oracle.sample(lg, oracle.Pcg32.seeded(0, 0), temperature=1.0, top_k=4)
    assert rc == 0 and list(ids) == [1, 2, 4, 0]
    # equal logits give bit-identical probabilities; the ordering keeps ids ascending among them
    assert probs[0] == probs[1] == probs[2] and probs[3] < probs[0]


def _fp64_probs(lg, k, temperature):
    order = sorted(range(len(lg)), key=lambda i: (-lg[i], i))[:k]
    z = np.array([lg[i] / temperature for i in order], np.float64)
    e = np.exp(z - z.max())
    return order, e / e.sum()


def test_probabilities_match_fp64_softmax():
    rng = np.random.default_rng(1)
    lg = (3 * rng.standard_normal(1000)).astype(np.float32)
    rc, _, ids, probs = oracle.sample(lg, oracle.Pcg32.seeded(9, 9), temperature=0.8, top_k=40)
    assert rc == 0
    order, ref = _fp64_probs(lg, 40, np.float32(0.8))
    assert list(ids) == order
    assert np.max(np.abs(probs - ref) / ref) < 1e-5


@pytest.mark.parametrize("top_p,keep", [(0.45, 1), (0.75, 2), (0.85, 3), (1.0, 3)])
def test_top_p_keeps_the_shortest_prefix_reaching_p(top_p, keep):
    lg = np.log(np.array([0.5, 0.3, 0.2], np.float64)).astype(np.float32)
    rc, _, ids, probs = oracle.sample(lg, oracle.Pcg32.seeded(5, 1), temperature=1.0, top_k=3, top_p=top_p)
    assert rc == 0 and len(ids) == keep and list(ids) == [0, 1, 2][:keep]
    assert abs(float(np.sum(probs, dtype=np.float64)) - 1.0) < 1e-6    # re-normalised prefix


def test_selection_is_the_first_cumulative_above_u():
    """Brute force: for each draw, recompute u from the same generator words and the cumulative sums of the
    returned probabilities; the token is the first index whose cumulative value exceeds u."""
    rng = np.random.default_rng(2)
    lg = rng.standard_normal(64).astype(np.float32)
    r = oracle.Pcg32.seeded(11, 4)
    shadow = oracle.Pcg32.seeded(11, 4)
    for _ in range(200):
        rc, tok, ids, probs = oracle.sample(lg, r, temperature=1.3, top_k=20, top_p=0.9)
        assert rc == 0
        u = oracle.pcg32_uniform(shadow.next())
        cum = np.cumsum(probs.astype(np.float64))
        j = int(np.searchsorted(cum, u, side="right"))
        j = min(j, len(ids) - 1)
        if min(abs(cum - u)) > 1e-6:     # away from a boundary the float and fp64 scans agree
            assert tok == ids[j]


def test_draw_frequencies_follow_the_distribution():
    """20000 draws at top-k 6, top-p 1: every token's frequency within 5 sigma of its fp64 probability."""
    lg = np.array([2.0, 1.5, 1.0, 0.0, -0.5, -3.0, -9.0], np.float32)
    order, ref = _fp64_probs(lg, 6, 1.0)
    r = oracle.Pcg32.seeded(2024, 7)
    n = 20000
    counts = np.zeros(len(lg))
    for _ in range(n):
        rc, tok, _, _ = oracle.sample(lg, r, temperature=1.0, top_k=6)
        assert rc == 0
        counts[tok] += 1
    assert counts[6] == 0                       # outside the top-k
    for i, p in zip(order, ref):
        assert abs(counts[i] / n - p) < 5 * math.sqrt(p * (1 - p) / n), (i, counts[i] / n, p)


def test_temperature_two_equals_halved_logits():
    """Dividing by 2 is exact, so temperature 2 and halved logits at temperature 1 draw identically."""
    rng = np.random.default_rng(3)
    lg = rng.standard_normal(300).astype(np.float32)
    a, b = oracle.Pcg32.seeded(8, 8), oracle.Pcg32.seeded(8, 8)
    for _ in range(50):
        ra, ta, _, _ = oracle.sample(lg, a, temperature=2.0, top_k=30, top_p=0.95)
        rb, tb, _, _ = oracle.sample(lg / np.float32(2), b, temperature=1.0, top_k=30, top_p=0.95)
        assert ra == rb == 0 and ta == tb


def test_masked_and_nan_tokens_are_never_drawn():
    lg = np.array([5.0, np.nan, 4.0, 6.0], np.float32)
    r = oracle.Pcg32.seeded(1, 1)
    for _ in range(100):
        rc, tok, _, _ = oracle.sample(lg, r, temperature=5.0, top_k=4, forbid=[3])
        assert rc == 0 and tok in (0, 2)


@pytest.mark.parametrize("kw,code", [
    (dict(penalty=0.0), 1), (dict(penalty=-1.0), 1), (dict(temperature=-1.0), 1), (dict(top_k=0), 1),
    (dict(top_p=0.0), 1), (dict(top_p=1.5), 1), (dict(temperature=np.inf), 1),
])
def test_invalid_parameters(kw, code):
    args = dict(temperature=1.0, top_k=5, top_p=1.0, penalty=1.0)
    args.update(kw)
    rc, _, _, _ = oracle.sample(np.zeros(8, np.float32), oracle.Pcg32.seeded(0, 0), **args)
    assert rc == code


def test_numerical_failures():
    r = oracle.Pcg32.seeded(0, 0)
    assert oracle.sample(np.full(4, -np.inf, np.float32), r)[0] == oracle.ORC_NUMERICAL_FAILURE
    assert oracle.sample(np.array([1.0, np.inf], np.float32), r)[0] == oracle.ORC_NUMERICAL_FAILURE
    assert oracle.sample(np.array([3e38, 1.0], np.float32), r, temperature=0.01)[0] == oracle.ORC_NUMERICAL_FAILURE
