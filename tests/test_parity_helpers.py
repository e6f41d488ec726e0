"""CPU checks of the parity helpers the GPU tests rely on."""
import numpy as np

from parity import bf16_to_f32, rel_l2


def test_bf16_widening_and_rel_l2():
    assert bf16_to_f32(np.uint16(0x4201)) - 32.0 == 0.25   # one bf16 ulp at 32
    assert bf16_to_f32(np.uint16(0xBF80)) == -1.0
    a = np.array([3.0, 4.0])
    assert rel_l2(a, a) == 0.0
    assert abs(rel_l2(np.array([3.0, 4.5]), a) - 0.1) < 1e-12


def _bf16_rne(x):
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def test_kv_gate_accepts_isolated_one_ulp_flips_only():
    """The KV teacher-forcing gate: isolated one-ulp rounding flips pass; a planted truncation (round toward
    zero instead of to nearest even, on one side) or a two-ulp error on an ordinary element fails; a
    near-zero element several ulps away but far below its row's scale passes."""
    import pytest
    from parity import bf16_order, kv_gate
    rng = np.random.default_rng(5)
    x = rng.standard_normal((2, 2, 8, 128)).astype(np.float32)   # [layer][K,V][kv head][dim]
    ref = _bf16_rne(x)
    g = ref.copy()
    g[0, 0, 3, 7] += 1
    g[1, 1, 0, 100] -= 1
    stats = {}
    assert kv_gate(g, ref, "t", stats) == 2 and stats["differ"] == 2 and stats["total"] == ref.size
    trunc = (x.view(np.uint32) >> 16).astype(np.uint16)
    with pytest.raises(AssertionError, match="differ"):
        kv_gate(ref, trunc, "t")
    g2 = ref.copy()
    big = int(np.argmax(np.abs(x[1, 1, 1])))
    g2[1, 1, 1, big] += 2
    with pytest.raises(AssertionError, match="ulps apart"):
        kv_gate(g2, ref, "t")
    near = ref.copy()
    near[0, 0, 2, 9] = _bf16_rne(np.float32(3e-6))
    near2 = near.copy()
    near2[0, 0, 2, 9] = _bf16_rne(np.float32(3.3e-6))
    assert kv_gate(near2, near, "t") == 1
    assert list(bf16_order(np.array([0x8001, 0x0000, 0x8000, 0x0001, 0x3F80, 0x3F81], np.uint16))) == [-1, 0, 0, 1,
                                                                                                        0x3F80, 0x3F81]
