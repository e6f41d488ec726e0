"""Host-side contract of libqw3 (no GPU needed): the library loads and exports every function the header
declares, and every host-detectable error returns its typed status before any device work.

Status numbering follows the error taxonomy of "Portable WebAssembly Runtime Architecture for TinyRustLM";
inventory rules (missing / mis-shaped / unexpected tensors, tied lm_head optional but byte-identical) follow
"M1 — Load the weights".
"""
import ctypes
import os
import re
from dataclasses import replace

import numpy as np
import pytest

import synth
import transformer_qwen3_block_amd as q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE_ARENA = 1 << 40  # aligned, never dereferenced by host-side calls


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(q._SO):
        q.build(force=False)
    return q.lib()


def cfg_of(shape, **over):
    kw = synth.abi_config_kwargs(shape)
    kw.update(over)
    return q.make_config(**kw)


SMALL = replace(synth.QWEN3_06B, vocab=1000, n_layers=2, n_q_heads=8, n_kv_heads=4, inter=1024, max_ctx=64,
                max_prefill=32)


def test_library_exports_every_declared_symbol(L):
    header = open(os.path.join(ROOT, "include", "qw3.h")).read()
    declared = set(re.findall(r"^\w[\w\s\*]*?\b(qw3_\w+)\s*\(", header, re.M))
    assert declared == set(q.EXPORTS), declared ^ set(q.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name
    assert L.qw3_abi_version() == q.ABI_VERSION


def test_preflight_sizes_follow_the_byte_model(L):
    for wl in synth.WORKLOADS:
        s = wl.shape
        sz = q.preflight(cfg_of(s))
        kv = 2 * s.n_seq * s.n_layers * s.n_kv_heads * s.max_ctx * s.head_dim * 2
        assert sz.kv == kv
        eb = 1 if s.fmt == synth.FMT_Q8 else 2
        mats = s.q_dim * s.hidden + 2 * s.kv_dim * s.hidden + s.hidden * s.q_dim + 3 * s.inter * s.hidden
        wbytes = s.n_layers * mats * eb + s.vocab * s.hidden * eb
        if s.fmt == synth.FMT_Q8:
            wbytes += (s.n_layers * mats + s.vocab * s.hidden) // 32 * 4
        assert sz.weights >= wbytes
        assert sz.total == sz.weights + sz.kv + sz.state + sz.scratch
    # the Q8 weight stream of the full model: 595,984,384 codes + 74,498,048 scale bytes
    s = synth.Q8_DECODE.shape
    mats = s.q_dim * s.hidden + 2 * s.kv_dim * s.hidden + s.hidden * s.q_dim + 3 * s.inter * s.hidden
    assert s.n_layers * mats + s.vocab * s.hidden == 595_984_384
    assert (s.n_layers * mats + s.vocab * s.hidden) // 32 * 4 == 74_498_048


@pytest.mark.parametrize("over,code", [
    (dict(abi_version=7), 2),
    (dict(head_dim=64), 13),
    (dict(n_q_heads=12, n_kv_heads=8), 13),     # 12 % 8 != 0
    (dict(n_q_heads=24, n_kv_heads=8), 13),     # group of 3: no kernel
    (dict(hidden=1280), 13),                    # not a multiple of 512 (bf16 lane slicing)
    (dict(n_seq=17), 13),
    (dict(weight_format=5), 12),
    (dict(weight_format=4, hidden=1536), 13),   # q8 x q8: contractions in multiples of 1024, as for Q8
    (dict(input_mode=1), 1),                    # hidden mode must have vocab 0
    (dict(vocab=0), 1),
    (dict(eps=0.0), 1),
    (dict(max_ctx=0), 1),
    (dict(theta=1.0), 1),
])
def test_preflight_rejects(L, over, code):
    sz = q.Sizes()
    assert L.qw3_preflight(ctypes.byref(cfg_of(SMALL, **over)), ctypes.byref(sz)) == code


def test_q8_needs_1024_multiples(L):
    sz = q.Sizes()
    c = cfg_of(replace(SMALL, fmt=synth.FMT_Q8, inter=1536))
    assert L.qw3_preflight(ctypes.byref(c), ctypes.byref(sz)) == 13
    assert L.qw3_preflight(None, ctypes.byref(sz)) == 1


def _create(L, cfg, arena=FAKE_ARENA, size=None):
    sz = q.preflight(cfg)
    h = ctypes.c_uint64(0)
    rc = L.qw3_create(ctypes.byref(cfg), ctypes.c_void_p(arena) if arena else None,
                      sz.total if size is None else size, ctypes.byref(h))
    return rc, h.value


def test_create_and_handle_lifecycle(L):
    cfg = cfg_of(SMALL)
    assert _create(L, cfg, arena=0)[0] == 1
    assert _create(L, cfg, arena=FAKE_ARENA + 8)[0] == 7
    assert _create(L, cfg, size=1000)[0] == 9
    rc, h = _create(L, cfg)
    assert rc == 0 and h >> 32 >= 1
    n = ctypes.c_int32(-1)
    assert L.qw3_get_len(h, 0, ctypes.byref(n)) == 0 and n.value == 0
    assert L.qw3_get_len(h, 1, ctypes.byref(n)) == 1
    assert L.qw3_reset_kv(h, 5) == 1 and L.qw3_reset_kv(h, -1) == 0
    # not loaded: stream-ordered calls are refused before any launch
    assert L.qw3_decode_step(h, ctypes.c_void_p(16), None, ctypes.c_void_p(16), None) == 1
    assert L.qw3_prefill(h, 0, ctypes.c_void_p(16), 4, None, None, None) == 1
    assert L.qw3_destroy(h) == 0
    assert L.qw3_destroy(h) == 5                       # stale
    assert L.qw3_get_len(h, 0, ctypes.byref(n)) == 5
    assert L.qw3_get_len((99 << 32) | 3, 0, ctypes.byref(n)) == 4
    assert L.qw3_get_len(0, 0, ctypes.byref(n)) == 4


def _tensor_array(tensors):
    arr = (q.Tensor * len(tensors))()
    keep = []
    for i, t in enumerate(tensors):
        data = np.ascontiguousarray(t["data"])
        sc = None if t.get("scales") is None else np.ascontiguousarray(t["scales"], np.float32)
        keep += [data, sc]
        rows, cols = (1, data.shape[0]) if data.ndim == 1 else data.shape
        if t["dtype"] == q.DT_Q8_0:
            cols = cols // 34 * 32
        arr[i] = q.Tensor(q.KIND[t["kind"]], t.get("layer", -1), t["dtype"], 0, rows, cols, data.ctypes.data,
                          sc.ctypes.data if sc is not None else None)
    return arr, keep


@pytest.fixture(scope="module")
def small_weights():
    return synth.make_weights(SMALL, seed=41)


@pytest.mark.parametrize("mutate", ["missing", "misshaped", "duplicate", "wrong_dtype", "bad_layer",
                                    "lm_head_differs", "unknown_kind"])
def test_load_weights_cross_check(L, small_weights, mutate):
    """Every inventory violation is InvalidModel, found before any device work (the arena is fake)."""
    tensors = synth.abi_tensors(small_weights)
    if mutate == "missing":
        tensors = [t for t in tensors if not (t["kind"] == "k_norm" and t["layer"] == 1)]
    elif mutate == "misshaped":
        t = next(t for t in tensors if t["kind"] == "down")
        t["data"] = t["data"][:, :-32]
    elif mutate == "duplicate":
        tensors.append(dict(tensors[3]))
    elif mutate == "wrong_dtype":
        t = next(t for t in tensors if t["kind"] == "q_norm")
        t["data"] = synth.bf16_to_f32(t["data"])
        t["dtype"] = q.DT_F32
    elif mutate == "bad_layer":
        next(t for t in tensors if t["kind"] == "o")["layer"] = 5
    elif mutate == "lm_head_differs":
        lm = small_weights.embed.bf16.copy()
        lm[3, 7] ^= 1
        tensors.append(dict(kind="lm_head", layer=-1, dtype=q.DT_BF16, data=lm))
    elif mutate == "unknown_kind":
        tensors[0] = dict(tensors[0])
    rc, h = _create(L, cfg_of(SMALL))
    assert rc == 0
    arr, keep = _tensor_array(tensors)
    if mutate == "unknown_kind":
        arr[0].kind = 42
    assert L.qw3_load_weights(h, arr, len(tensors), None) == 10
    assert L.qw3_destroy(h) == 0


def test_hidden_mode_rejects_global_tensors(L):
    shp = replace(synth.SINGLE_BLOCK.shape, max_ctx=16)
    W = synth.make_weights(shp, seed=42)
    tensors = synth.abi_tensors(W)
    tensors.append(dict(kind="final_norm", layer=-1, dtype=q.DT_BF16, data=W.layers[0]["attn_norm"]))
    rc, h = _create(L, cfg_of(shp))
    assert rc == 0
    arr, keep = _tensor_array(tensors)
    assert L.qw3_load_weights(h, arr, len(tensors), None) == 10
    L.qw3_destroy(h)


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(q, "_SO", str(tmp_path / "missing.so"))
    monkeypatch.setattr(q, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        q.lib()


def test_rope_table_bit_exact_with_oracle(L):
    """The table the library uploads equals the oracle's (angle, cos, sin in double, one rounding to f32) bit
    for bit at every position of a long context, including positions where an f32 angle would differ."""
    import oracle
    theta, n = 1e6, 8300
    c, s = q.rope_table(theta, 128, n)
    for pos in list(range(0, 64)) + list(range(2040, 2060)) + list(range(8180, 8300)):
        oc, os_ = oracle.rope_table(theta, 128, pos)
        assert np.array_equal(c[pos].view(np.uint32), oc.view(np.uint32)), pos
        assert np.array_equal(s[pos].view(np.uint32), os_.view(np.uint32)), pos
    assert np.all(c[0] == 1.0) and np.all(s[0] == 0.0)
    with pytest.raises(q.Qw3Error):
        q.rope_table(1.0, 128, 4)


def test_bf16_single_token_tiles_are_accepted(L):
    """A bf16 model whose prefill tile is one token has no MFMA prefill; it is still a valid configuration
    (prompts run token by token through the decode kernels)."""
    sz = q.preflight(cfg_of(replace(SMALL, max_prefill=1)))
    assert sz.total > 0
    h = ctypes.c_uint64(0)
    assert L.qw3_create(ctypes.byref(cfg_of(replace(SMALL, max_prefill=1))), ctypes.c_void_p(FAKE_ARENA),
                        sz.total, ctypes.byref(h)) == 0
    assert L.qw3_destroy(h.value) == 0


@pytest.mark.parametrize("mutate", ["q8_codes_for_q8_0", "scales_given", "nan_scale", "short_blocks",
                                    "lm_head_differs"])
def test_q8_0_inventory_cross_check(L, mutate):
    """The Q8_0 format takes the pages' 34-byte blocks: another quantized layout, extra scales, a non-finite
    f16 scale, truncated blocks or a differing tied lm_head are InvalidModel before any device work."""
    shp = replace(SMALL, fmt=synth.FMT_Q8_0)
    W = synth.make_weights(shp, seed=43)
    tensors = synth.abi_tensors(W)
    assert all(t["dtype"] == q.DT_Q8_0 for t in tensors if t["kind"] in ("q", "embed", "down"))
    t = next(t for t in tensors if t["kind"] == "gate" and t["layer"] == 1)
    if mutate == "q8_codes_for_q8_0":
        t.update(dtype=q.DT_Q8, data=W.layers[1]["gate"].codes, scales=W.layers[1]["gate"].scales)
    elif mutate == "scales_given":
        t["scales"] = W.layers[1]["gate"].scales
    elif mutate == "nan_scale":
        blk = t["data"].copy()
        blk[5, 34 * 3 + 1] = 0x7E   # f16 0x7Exx: NaN
        t["data"] = blk
    elif mutate == "short_blocks":
        t["data"] = t["data"][:, :-34]
    elif mutate == "lm_head_differs":
        lm = W.embed.q8_0.copy()
        lm[2, 40] ^= 1
        tensors.append(dict(kind="lm_head", layer=-1, dtype=q.DT_Q8_0, data=lm))
    rc, h = _create(L, cfg_of(shp))
    assert rc == 0
    arr, keep = _tensor_array(tensors)
    assert L.qw3_load_weights(h, arr, len(tensors), None) == 10
    L.qw3_destroy(h)
