"""Shared helpers of the GPU parity tests: model construction from synthetic weights, the tolerance
check and the greedy-token comparison rule.

Tolerance: every compared logits or hidden-state vector must satisfy BOTH max-abs <= 2e-2 and relative
L2 (||gpu - ref|| / ||ref||) <= 1e-2 against the oracle.  Integer results (dequantised weights, KV-cache
contents, argmax ids) are compared bit for bit; an argmax may differ from the oracle's only when the
oracle's own top-1/top-2 margin is smaller than twice the observed max-abs logit difference of that step
(then both ids are correct within the tolerance), and exact ties must pick the lowest id.

Decode trajectories are compared with the KV cache teacher-forced (sync_appended_kv): the appended bf16 K/V
of every step must be within the relative-L2 tolerance of the oracle's, and the oracle continues from the
GPU's cache.
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


def bf16_to_f32(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def sync_appended_kv(gpu_model, orc, seq, pos, n_layers, orc_seq=None):
    """KV teacher forcing.  Both sides round the appended K and V to bf16; two correct f32 evaluations in
    different summation orders can land on opposite sides of a bf16 rounding boundary (one ulp, 0.4 %), a flip
    in one layer moves the later layers' K/V of the same position, and a free-running comparison then drifts
    for every later step.  So after a step each layer's appended K and V are checked against the oracle's
    (relative L2 within the hidden-state tolerance: an index, head or position error is an O(1) difference)
    and the oracle's copy is replaced by the GPU's: every step is compared from the same cache.  Returns the
    number of appended elements that differ."""
    oseq = seq if orc_seq is None else orc_seq
    differ = 0
    for l in range(n_layers):
        gk, gv = gpu_model.kv_read(seq, l, pos, 1)
        gk = gk.cpu().numpy().view(np.uint16)
        gv = gv.cpu().numpy().view(np.uint16)
        rc, ok_, ov = orc.kv_read(oseq, l, pos, 1)
        assert rc == 0
        for g_, o_, nm in ((gk, ok_, "K"), (gv, ov, "V")):
            r = rel_l2(bf16_to_f32(g_), bf16_to_f32(o_))
            assert r <= REL_L2, f"appended {nm} of layer {l} at position {pos}: rel-L2 {r:.3e}"
            differ += int(np.count_nonzero(g_ != o_))
        assert orc.kv_write(oseq, l, pos, gk, gv) == 0
    return differ


def build_gpu_model(W, device="cuda:0", with_lm_head=False):
    import synth
    import transformer_qwen3_block_amd as q
    cfg = q.make_config(**synth.abi_config_kwargs(W.shape))
    m = q.Model(cfg, device=device)
    m.load_weights(synth.abi_tensors(W, with_lm_head=with_lm_head))
    return m
