"""Shared helpers of the GPU parity tests: model construction from synthetic weights, the tolerance
check and the greedy-token comparison rule.

Tolerance: every compared logits or hidden-state vector must satisfy BOTH max-abs <= 2e-2 and relative
L2 (||gpu - ref|| / ||ref||) <= 1e-2 against the oracle.  Integer results (dequantised weights, KV-cache
contents, argmax ids) are compared bit for bit; an argmax may differ from the oracle's only when the
oracle's own top-1/top-2 margin is smaller than twice the observed max-abs logit difference of that step
(then both ids are correct within the tolerance), and exact ties must pick the lowest id.

Decode trajectories are compared with the KV cache teacher-forced (forced_step): every appended bf16 K/V
element must equal the oracle's own rounding, sit one bf16 ulp from it, or (near zero) differ by at most 2^-10
of its head row's RMS; at most 5 % of a step's elements may differ; and the oracle's step uses the GPU's
appended values, so both sides attend over the same cache.  A prompt's whole cache is forced the same way
after a prefill (sync_prefilled_kv).
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


# At most this fraction of a step's appended bf16 K/V elements may differ from the oracle's.  Two correct f32
# evaluations in different summation orders round to different bf16 values with probability about
# |f32 difference| / (bf16 ulp) per element; with the current position teacher-forced (forced_step) the
# measured rates are 0.05-0.3 % at 1-2 layers and at most 0.73 % at 28 layers.  A systematic error such as
# truncation instead of round-to-nearest-even moves about half of them.
KV_FLIP_FRACTION = 0.05
# Each differing element is one bf16 ulp from the oracle's, or -- for an element near zero, where rotation
# and normalisation cancel large terms and a tiny absolute difference spans several ulps of a tiny value --
# within this fraction of the RMS of its 128-wide head row.
KV_NEAR_ZERO = 2.0 ** -10


def bf16_order(bits):
    """bf16 bit patterns mapped to integers in value order (adjacent representable values differ by 1)."""
    b = np.asarray(bits, np.uint16).astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def read_appended_kv(gpu_model, seq, pos, n_layers):
    """The GPU's appended bf16 K/V bits of one position: uint16 [n_layers][2][n_kv_heads][head_dim]."""
    out = None
    for l in range(n_layers):
        gk, gv = gpu_model.kv_read(seq, l, pos, 1)
        gk = gk.cpu().numpy().view(np.uint16)[:, 0]
        gv = gv.cpu().numpy().view(np.uint16)[:, 0]
        if out is None:
            out = np.empty((n_layers, 2) + gk.shape, np.uint16)
        out[l, 0], out[l, 1] = gk, gv
    return out


def kv_gate(gpu_bits, orc_bits, where, stats=None):
    """The appended K/V of one position, GPU against the oracle's own rounding ([L][2][HKV][D] bf16 bits):
    every element equal, one bf16 ulp apart or (near zero) within KV_NEAR_ZERO of its head row's RMS, and at
    most KV_FLIP_FRACTION of the elements apart.  Returns the number that differ."""
    d = np.abs(bf16_order(gpu_bits) - bf16_order(orc_bits))
    gf = bf16_to_f32(gpu_bits).astype(np.float64)
    of = bf16_to_f32(orc_bits).astype(np.float64)
    rms = np.sqrt(np.mean(of * of, axis=-1, keepdims=True))
    bad = (d > 1) & (np.abs(gf - of) > KV_NEAR_ZERO * rms)
    if bad.any():
        l, kv, h, e = (int(i[0]) for i in np.nonzero(bad))
        raise AssertionError(f"{where}: appended {'KV'[kv]} of layer {l}, head {h}, dim {e}: {int(d[l, kv, h, e])} "
                             f"bf16 ulps apart ({gf[l, kv, h, e]:.6g} vs {of[l, kv, h, e]:.6g}, head RMS "
                             f"{float(rms[l, kv, h, 0]):.3g})")
    differ, total = int(np.count_nonzero(d)), int(d.size)
    assert differ <= KV_FLIP_FRACTION * total, f"{where}: {differ} of {total} appended K/V elements differ"
    if stats is not None:
        stats["differ"] = stats.get("differ", 0) + differ
        stats["total"] = stats.get("total", 0) + total
        stats["worst"] = max(stats.get("worst", 0.0), differ / total)
    return differ


def forced_step(gpu_model, orc, seq, tok, n_layers, orc_seq=None, stats=None):
    """KV teacher forcing.  Both sides round the appended K and V to bf16, and two correct f32 evaluations in
    different summation orders can land on opposite sides of a bf16 rounding boundary.  Attention reads the
    new position within the same step (its own weight can be large), and the cache keeps it for every later
    step, so a flip moves everything after it.  So the oracle's step for the position the GPU just appended
    takes the GPU's bf16 K/V there (its arithmetic otherwise unchanged), after the oracle's own rounding of
    the same values passed kv_gate.  Run after the GPU step; returns the oracle's (rc, argmax, logits,
    hidden)."""
    oseq = seq if orc_seq is None else orc_seq
    pos = orc.get_len(oseq)
    g = read_appended_kv(gpu_model, seq, pos, n_layers)
    rc, am, lg, hid, own = orc.step_forced(oseq, tok, kv_force=g)
    if rc == 0:
        kv_gate(g, own, f"position {pos}", stats)
    return rc, am, lg, hid


# The q8 x q8 format's deep tier (two or more layers).  Its activation codes are integers decided on f32 inputs
# that differ from the oracle's by reassociation only; a code that lands on the other side of a rounding
# boundary moves its input by one quantization step (max|x|/127 of the block), and the layers after it amplify
# that.  So past one layer the comparison is the pages' conformance measures per step: the greedy choice (equal,
# or a near-tie within the observed logit difference) and the cosine similarity of the logits.
ACT8_COS = 0.99
ACT8_KV_REL = 0.1


def cosine(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.dot(a, b) / max(np.linalg.norm(a) * np.linalg.norm(b), 1e-300))


def forced_step_act8(gpu_model, orc, seq, tok, n_layers, orc_seq=None, stats=None):
    """forced_step for the deep q8 x q8 tier: the GPU's appended K/V (of every layer, within ACT8_KV_REL
    relative L2 of the oracle's own) replaces the oracle's for this step."""
    oseq = seq if orc_seq is None else orc_seq
    pos = orc.get_len(oseq)
    g = read_appended_kv(gpu_model, seq, pos, n_layers)
    rc, am, lg, hid, own = orc.step_forced(oseq, tok, kv_force=g)
    if rc == 0:
        worst = max(rel_l2(bf16_to_f32(g[l]), bf16_to_f32(own[l])) for l in range(n_layers))
        assert worst <= ACT8_KV_REL, f"position {pos}: appended K/V rel-L2 {worst:.3e}"
        if stats is not None:
            stats["kv_rel"] = max(stats.get("kv_rel", 0.0), worst)
    return rc, am, lg, hid


def sync_prefilled_kv(gpu_model, orc, seq, n_pos, n_layers, orc_seq=None):
    """KV teacher forcing of a whole prompt.  The tiled prefill feeds MFMA f16 operands, so its cache is close
    to the oracle's (relative L2 within the hidden-state tolerance per layer) but not one-ulp close; decode
    steps after it are compared from the same cache, so the GPU's prompt cache replaces the oracle's."""
    oseq = seq if orc_seq is None else orc_seq
    worst = 0.0
    for l in range(n_layers):
        gk, gv = gpu_model.kv_read(seq, l, 0, n_pos)
        gk = gk.cpu().numpy().view(np.uint16)
        gv = gv.cpu().numpy().view(np.uint16)
        rc, ok_, ov = orc.kv_read(oseq, l, 0, n_pos)
        assert rc == 0
        for g_, o_, nm in ((gk, ok_, "K"), (gv, ov, "V")):
            r = rel_l2(bf16_to_f32(g_), bf16_to_f32(o_))
            assert r <= REL_L2, f"prompt {nm} cache of layer {l}: rel-L2 {r:.3e}"
            worst = max(worst, r)
        assert orc.kv_write(oseq, l, 0, gk, gv) == 0
    return worst


class Margins:
    """Worst max-abs / relative-L2 over the compared vectors of one test, printed at the end."""

    def __init__(self, what):
        self.what, self.mab, self.rel, self.n = what, 0.0, 0.0, 0

    def add(self, mab_rel):
        self.mab = max(self.mab, mab_rel[0])
        self.rel = max(self.rel, mab_rel[1])
        self.n += 1

    def report(self, kv=None):
        extra = ""
        if kv and kv.get("total"):
            extra = (f"; appended K/V elements that differ from the oracle's: {kv['differ']} of {kv['total']}, "
                     f"worst step {100 * kv.get('worst', 0):.2f} %")
        print(f"MARGIN {self.what}: {self.n} vectors, worst max-abs {self.mab:.3e} (bound {MAX_ABS}), worst rel-L2 "
              f"{self.rel:.3e} (bound {REL_L2}){extra}", flush=True)


def build_gpu_model(W, device="cuda:0", with_lm_head=False):
    import synth
    import transformer_qwen3_block_amd as q
    cfg = q.make_config(**synth.abi_config_kwargs(W.shape))
    m = q.Model(cfg, device=device)
    m.load_weights(synth.abi_tensors(W, with_lm_head=with_lm_head))
    return m
