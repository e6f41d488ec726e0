"""Shared helpers of the GPU parity tests: model construction from synthetic weights, the tolerance
check and the greedy-token comparison rule.

Tolerance: every compared logits or hidden-state vector must satisfy BOTH max-abs <= 2e-2 and relative
L2 (||gpu - ref|| / ||ref||) <= 1e-2 against the oracle.  Integer results (dequantised weights, KV-cache
contents, argmax ids) are compared bit for bit; an argmax may differ from the oracle's only when the
oracle's own top-1/top-2 margin is smaller than twice the observed max-abs logit difference of that step
(then both ids are correct within the tolerance), and exact ties must pick the lowest id.
"""
import numpy as np

MAX_ABS = 2e-2
REL_L2 = 1e-2


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def assert_close(gpu, ref, what="", max_abs=MAX_ABS, rel=REL_L2):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU values"
    mab = float(np.max(np.abs(gpu - ref))) if gpu.size else 0.0
    r = rel_l2(gpu, ref)
    assert mab <= max_abs and r <= rel, f"{what}: max-abs {mab:.3e} (<= {max_abs}), rel-L2 {r:.3e} (<= {rel})"
    return mab, r


def argmax_ok(gpu_id, ref_logits, gpu_logits=None):
    """True when gpu_id is the oracle's greedy choice, or a near-tie the tolerance cannot separate."""
    ref_logits = np.asarray(ref_logits, np.float32)
    ref_id = int(np.argmax(ref_logits))
    if gpu_id == ref_id:
        return True
    if gpu_logits is None:
        return False
    diff = float(np.max(np.abs(np.asarray(gpu_logits, np.float64) - ref_logits)))
    top = np.sort(ref_logits)[::-1]
    margin = float(top[0] - ref_logits[gpu_id])
    return margin < 2 * diff


def build_gpu_model(W, device="cuda:0", with_lm_head=False):
    import synth
    import transformer_qwen3_block_amd as q
    cfg = q.make_config(**synth.abi_config_kwargs(W.shape))
    m = q.Model(cfg, device=device)
    m.load_weights(synth.abi_tensors(W, with_lm_head=with_lm_head))
    return m
