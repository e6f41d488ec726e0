"""CPU checks of the parity helpers the GPU tests rely on."""
import numpy as np

from parity import bf16_to_f32, rel_l2


def test_bf16_widening_and_rel_l2():
    assert bf16_to_f32(np.uint16(0x4201)) - 32.0 == 0.25   # one bf16 ulp at 32
    assert bf16_to_f32(np.uint16(0xBF80)) == -1.0
    a = np.array([3.0, 4.0])
    assert rel_l2(a, a) == 0.0
    assert abs(rel_l2(np.array([3.0, 4.5]), a) - 0.1) < 1e-12
