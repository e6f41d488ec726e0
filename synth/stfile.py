"""A minimal writer of safetensors containers: synthetic weight files for the loader tests and the loader's
benchmark line (test and benchmark infrastructure, like the rest of this package).

Layout ("Scalar-Native Qwen3 Reference Runtime As The Numerical Authority", section 3 "File Layout and Safe
Metadata Parsing"; "M1 — Load the weights", "The safetensors format -- three regions"): an 8-byte little-endian
header length, the JSON header, then the data blob.  The header is padded with spaces so the blob starts on an
8-byte boundary, and tensors are laid out back to back in the order given, each padded to a multiple of 8
bytes by the next tensor's start -- unless a test asks for something else.  Its output is checked against the
`safetensors` package's reader in the tests.
"""
import json
import struct

import numpy as np

QWEN3_BLOCK = (("input_layernorm.weight", "attn_norm"), ("self_attn.q_proj.weight", "q"),
               ("self_attn.k_proj.weight", "k"), ("self_attn.v_proj.weight", "v"),
               ("self_attn.q_norm.weight", "q_norm"), ("self_attn.k_norm.weight", "k_norm"),
               ("self_attn.o_proj.weight", "o"), ("post_attention_layernorm.weight", "mlp_norm"),
               ("mlp.gate_proj.weight", "gate"), ("mlp.up_proj.weight", "up"), ("mlp.down_proj.weight", "down"))


def write(path, entries, metadata=None, header_extra=b"", blob_override=None, sparse_blob=None):
    """entries: list of (name, dtype, shape, raw bytes or None, begin override, end override).  Returns the
    header dict written.  With sparse_blob=N the blob is N bytes of zeros left as a hole in the file."""
    header = {}
    if metadata is not None:
        header["__metadata__"] = metadata
    at = 0
    blobs = []
    for name, dtype, shape, raw, b_ov, e_ov in entries:
        n = len(raw) if raw is not None else _nbytes(dtype, shape)
        begin = at if b_ov is None else b_ov
        end = begin + n if e_ov is None else e_ov
        header[name] = {"dtype": dtype, "shape": list(shape), "data_offsets": [begin, end]}
        if raw is not None:
            blobs.append((begin, raw))
        at = (begin + n + 7) // 8 * 8
    h = json.dumps(header, separators=(",", ":")).encode() + header_extra
    h += b" " * ((8 - (8 + len(h)) % 8) % 8)
    with open(path, "wb") as f:
        f.write(struct.pack("<Q", len(h)))
        f.write(h)
        if sparse_blob is not None:
            f.truncate(8 + len(h) + sparse_blob)
        else:
            total = at if blob_override is None else blob_override
            buf = bytearray(total)
            for b, raw in blobs:
                buf[b:b + len(raw)] = raw[:max(0, total - b)]
            f.write(bytes(buf))
    return header


def _nbytes(dtype, shape):
    n = int(np.prod(shape, dtype=np.int64)) if shape else 1
    if dtype == "Q8_0":
        return shape[0] * (shape[1] // 32) * 34
    return n * {"BF16": 2, "F32": 4, "I8": 1}[dtype]


def model_entries(W, with_lm_head=True):
    """The Qwen3 inventory of a synth.Weights: bf16 models as BF16, Q8_0 models as Q8_0 blocks + F32 norms."""
    import synth
    q = W.shape.fmt == synth.FMT_Q8_0
    assert W.shape.fmt in (synth.FMT_BF16, synth.FMT_Q8_0)

    def mat(m):
        return ("Q8_0", m.q8_0.tobytes()) if q else ("BF16", m.bf16.tobytes())

    def vec(v):
        return ("F32", np.asarray(v, np.float32).tobytes()) if q else ("BF16", np.asarray(v, np.uint16).tobytes())

    out = []
    dt, raw = mat(W.embed)
    out.append(("model.embed_tokens.weight", dt, [W.embed.rows, W.embed.cols], raw, None, None))
    for l, d in enumerate(W.layers):
        for name, slot in QWEN3_BLOCK:
            v = d[slot]
            if slot in synth.MATRIX_SLOTS:
                dt, raw = mat(v)
                shape = [v.rows, v.cols]
            else:
                dt, raw = vec(v)
                shape = [len(v)]
            out.append((f"model.layers.{l}.{name}", dt, shape, raw, None, None))
    dt, raw = vec(W.final_norm)
    out.append(("model.norm.weight", dt, [len(W.final_norm)], raw, None, None))
    if with_lm_head:
        dt, raw = mat(W.embed)
        out.append(("lm_head.weight", dt, [W.embed.rows, W.embed.cols], raw, None, None))
    return out
