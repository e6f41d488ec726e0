"""Host-side checks of the weight-file reader (qw3_inspect_file): the safetensors / SLM2 container rules of
"Scalar-Native Qwen3 Reference Runtime As The Numerical Authority" section 3 ("File Layout and Safe Metadata
Parsing": file boundary, non-overlapping sequential spans, 8-byte alignment) and "M1 — Load the weights"
(parse_tensor_entry size rule, the expected inventory, stored / logical / embedding parameter counts).  No GPU:
the reader maps and validates the file without touching a device.
"""
import json
import os
import struct
from dataclasses import replace

import numpy as np
import pytest

from synth import stfile
import synth
import transformer_qwen3_block_amd as q

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
TINY = replace(synth.QWEN3_06B, vocab=96, n_layers=2, n_q_heads=8, n_kv_heads=4, inter=1024, max_ctx=32)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(q._SO):
        q.build(force=False)
    return q.lib()


def _code(L, path):
    r = q.FileReport()
    return L.qw3_inspect_file(os.fsencode(str(path)), r), r


def test_qwen3_inventory_counts_from_the_pages(L, tmp_path):
    """A Qwen3-0.6B-shaped bf16 header (blob left as a sparse hole): 311 tensors, 751,632,384 stored,
    596,049,920 logical and 155,582,464 embedding parameters, as printed on the pages."""
    g = json.load(open(os.path.join(GOLDEN, "qwen3_06b_inventory.json")))
    s = synth.QWEN3_06B
    shapes = {"attn_norm": [s.hidden], "mlp_norm": [s.hidden], "q_norm": [s.head_dim], "k_norm": [s.head_dim]}
    ents = [("model.embed_tokens.weight", "BF16", [s.vocab, s.hidden], None, None, None)]
    for l in range(s.n_layers):
        for name, slot in stfile.QWEN3_BLOCK:
            shp = shapes.get(slot) or list(s.matrix_shape(slot))
            ents.append((f"model.layers.{l}.{name}", "BF16", shp, None, None, None))
    ents.append(("model.norm.weight", "BF16", [s.hidden], None, None, None))
    ents.append(("lm_head.weight", "BF16", [s.vocab, s.hidden], None, None, None))
    blob = sum((stfile._nbytes(e[1], e[2]) + 7) // 8 * 8 for e in ents)
    p = tmp_path / "qwen3.safetensors"
    stfile.write(p, ents, metadata={"format": "pt"}, sparse_blob=blob)
    rc, r = _code(L, p)
    assert rc == 0
    assert r.n_tensors == g["tensor_count"]["value"]
    assert r.stored_params == g["params_stored"]["value"]
    assert r.logical_params == g["params_logical"]["value"]
    assert r.embed_params == g["params_embeddings"]["value"]
    assert r.n_layers == 28 and r.lm_head_present == 1


@pytest.mark.parametrize("fmt", [synth.FMT_BF16, synth.FMT_Q8_0])
def test_writer_output_reads_back_through_the_reference_reader(L, tmp_path, fmt):
    """The test writer's files are what the `safetensors` package reads (pins the writer), and a file the
    package writes itself passes the library's reader with the right counts."""
    import torch
    from safetensors import safe_open
    from safetensors.torch import save_file
    W = synth.make_weights(replace(TINY, fmt=fmt), seed=61)
    ents = stfile.model_entries(W)
    p = tmp_path / "m.safetensors"
    stfile.write(p, ents)
    assert _code(L, p)[0] == 0
    if fmt == synth.FMT_BF16:
        with safe_open(str(p), framework="pt") as f:
            t = f.get_tensor("model.layers.1.mlp.down_proj.weight")
            assert t.dtype == torch.bfloat16
            assert np.array_equal(t.view(torch.int16).numpy().view(np.uint16), W.layers[1]["down"].bf16)
        tensors = {e[0]: torch.from_numpy(np.frombuffer(e[3], np.int16).reshape(e[2]).copy()).view(torch.bfloat16)
                   for e in ents}
        p2 = tmp_path / "ref.safetensors"
        save_file(tensors, str(p2))
        rc, r = _code(L, p2)
        assert rc == 0 and r.n_tensors == len(ents) and r.lm_head_present == 1
    else:
        # the reference reader parses the container's header; Q8_0 is this format's own dtype (an SLM2 file)
        hdr_len = struct.unpack("<Q", open(p, "rb").read(8))[0]
        hdr = json.loads(open(p, "rb").read(8 + hdr_len)[8:])
        assert hdr["model.layers.0.self_attn.q_proj.weight"]["dtype"] == "Q8_0"


def _one(name="model.norm.weight", dtype="F32", shape=(64,), raw=None, b=None, e=None):
    raw = raw if raw is not None else np.zeros(int(np.prod(shape)), np.float32).tobytes()
    return (name, dtype, list(shape), raw, b, e)


@pytest.mark.parametrize("case,code", [
    ("ok", 0), ("unknown_name", 10), ("unknown_dtype", 10), ("size_mismatch", 10), ("end_beyond_blob", 6),
    ("overlap", 10), ("hole", 10), ("trailing", 10), ("misaligned", 7), ("duplicate_key", 10),
    ("negative", 10), ("fraction", 10), ("overflow", 8), ("metadata_not_string", 10), ("bad_json", 10),
    ("header_beyond_file", 6), ("extra_field", 10), ("q8_0_partial_block", 10), ("layer_leading_zero", 10),
])
def test_header_rules(L, tmp_path, case, code):
    p = tmp_path / f"{case}.safetensors"
    a = _one()
    b = _one("model.layers.0.input_layernorm.weight")
    ents = [a, b]
    kw = {}
    if case == "unknown_name":
        ents = [a, _one("model.layers.0.attn.weird")]
    elif case == "unknown_dtype":
        ents = [a, _one("model.layers.0.input_layernorm.weight", dtype="F16")]
    elif case == "size_mismatch":
        ents = [a, _one("model.layers.0.input_layernorm.weight", shape=(63,), raw=bytes(256))]
    elif case == "end_beyond_blob":
        ents = [a, _one("model.layers.0.input_layernorm.weight", b=256, e=256 + 256 + 64)]
        kw["blob_override"] = 512
    elif case == "overlap":
        ents = [a, _one("model.layers.0.input_layernorm.weight", b=128, e=384)]
    elif case == "hole":
        ents = [a, _one("model.layers.0.input_layernorm.weight", b=264, e=520)]
        kw["blob_override"] = 520
    elif case == "trailing":
        kw["blob_override"] = 512 + 8
    elif case == "misaligned":
        ents = [_one(raw=bytes(256), shape=(64,)), _one("model.layers.0.input_layernorm.weight", dtype="BF16",
                                                         shape=(3,), raw=bytes(6), b=256, e=262),
                _one("model.layers.0.post_attention_layernorm.weight", dtype="BF16", shape=(1,), raw=bytes(2),
                     b=262, e=264)]
    elif case == "layer_leading_zero":
        ents = [a, _one("model.layers.01.input_layernorm.weight")]
    stfile.write(p, ents, **kw)
    raw = bytearray(open(p, "rb").read())
    n = struct.unpack("<Q", raw[:8])[0]
    hdr = raw[8:8 + n].decode()

    def rewrite(new_hdr):
        new_hdr = new_hdr.encode()
        new_hdr += b" " * ((8 - (8 + len(new_hdr)) % 8) % 8)
        open(p, "wb").write(struct.pack("<Q", len(new_hdr)) + new_hdr + bytes(raw[8 + n:]))

    if case == "duplicate_key":
        rewrite(hdr.rstrip()[:-1] + ',"model.norm.weight":' + json.dumps(json.loads(hdr)["model.norm.weight"]) + "}")
    elif case == "negative":
        rewrite(hdr.replace('"shape":[64]', '"shape":[-64]', 1))
    elif case == "fraction":
        rewrite(hdr.replace('"shape":[64]', '"shape":[64.0]', 1))
    elif case == "overflow":
        rewrite(hdr.replace('"shape":[64]', '"shape":[99999999999999999999]', 1))
    elif case == "metadata_not_string":
        rewrite('{"__metadata__":{"a":1},' + hdr.strip()[1:])
    elif case == "bad_json":
        rewrite(hdr.strip()[:-1])
    elif case == "header_beyond_file":
        open(p, "wb").write(struct.pack("<Q", 10 ** 6) + bytes(raw[8:]))
    elif case == "extra_field":
        rewrite(hdr.replace('"dtype":"F32"', '"dtype":"F32","offset":0', 1))
    elif case == "q8_0_partial_block":
        ents = [("model.layers.0.self_attn.q_proj.weight", "Q8_0", [2, 48], bytes(2 * 2 * 34), None, None)]
        stfile.write(p, ents)
    assert _code(L, p)[0] == code


def test_unreadable_path(L, tmp_path):
    assert _code(L, tmp_path / "nope.safetensors")[0] == 1


@pytest.mark.parametrize("file_fmt,cfg_fmt,over", [(synth.FMT_BF16, synth.FMT_Q8_0, {}),
                                                    (synth.FMT_Q8_0, synth.FMT_BF16, {}),
                                                    (synth.FMT_BF16, synth.FMT_BF16, {"n_layers": 3})])
def test_file_that_does_not_match_the_configuration(L, tmp_path, file_fmt, cfg_fmt, over):
    """A valid container whose tensors do not fit the handle's configuration (another weight format, a
    missing layer) is InvalidModel from the cross-check, before any device work (the arena is fake)."""
    import ctypes
    W = synth.make_weights(replace(TINY, fmt=file_fmt), seed=62)
    p = tmp_path / "m.safetensors"
    stfile.write(p, stfile.model_entries(W, with_lm_head=False))
    cfg = q.make_config(**synth.abi_config_kwargs(replace(TINY, fmt=cfg_fmt, **over)))
    sz = q.preflight(cfg)
    h = ctypes.c_uint64(0)
    assert L.qw3_create(ctypes.byref(cfg), ctypes.c_void_p(1 << 40), sz.total, ctypes.byref(h)) == 0
    assert L.qw3_load_file(h.value, os.fsencode(str(p)), None) == 10
    L.qw3_destroy(h.value)
