"""GPU: weights loaded from a safetensors (bf16) or SLM2 (Q8_0 blocks + f32 norms) file through
qw3_load_file decode exactly like the same tensors handed to qw3_load_weights (bit-identical logits), with and
without the tied lm_head copy ("M1 — Load the weights", "Tied != absent")."""
from dataclasses import replace

import numpy as np
import pytest

from synth import stfile
import synth
from parity import build_gpu_model

pytestmark = pytest.mark.gpu

SMALL = replace(synth.QWEN3_06B, vocab=1000, n_layers=2, n_q_heads=8, n_kv_heads=4, inter=1024, max_ctx=64,
                max_prefill=16)


@pytest.mark.parametrize("fmt", [synth.FMT_BF16, synth.FMT_Q8_0])
@pytest.mark.parametrize("lm_head", [True, False])
def test_file_load_equals_tensor_load(tmp_path, fmt, lm_head):
    import torch
    import transformer_qwen3_block_amd as q
    shp = replace(SMALL, fmt=fmt)
    W = synth.make_weights(shp, seed=63)
    p = tmp_path / ("m.safetensors" if fmt == synth.FMT_BF16 else "m.slm2")
    stfile.write(p, stfile.model_entries(W, with_lm_head=lm_head), metadata={"format": "pt"})
    rep = q.inspect_file(p)
    assert rep.n_tensors == 2 + 11 * shp.n_layers + (1 if lm_head else 0)
    a = build_gpu_model(W)
    b = q.Model(q.make_config(**synth.abi_config_kwargs(shp)))
    b.load_file(p)
    toks = torch.from_numpy(synth.tokens(63, 0, 9, shp.vocab)).cuda()
    outs = []
    for m in (a, b):
        lg = torch.empty((1, shp.vocab), dtype=torch.float32, device="cuda")
        am = torch.empty(1, dtype=torch.int32, device="cuda")
        m.prefill(toks[:8].contiguous(), 0, None, am)
        m.decode_step(toks[8:9].contiguous(), am, lg)
        torch.cuda.synchronize()
        outs.append(lg.cpu().numpy())
        assert m.status() == 0
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
