"""Oracle for the Qwen3 decoder-block forward pass (strict f32, token by token, on the CPU).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, the smoke check and the benchmark's
``cpu_baseline`` leg may import this package; the product library never links
or calls it.  The C source (``orc.c``) holds the arithmetic; this module is a
ctypes binding plus the fp64 matrix-form twin used to pin it (``twin64.py``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liborc.so")

ORC_OK, ORC_INVALID_ARGUMENT, ORC_CONTEXT_EXCEEDED, ORC_NUMERICAL_FAILURE = 0, 1, 14, 18
# Strict lane: no FMA contraction, no fast math, no host-specific vector ISA.
CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fno-unsafe-math-optimizations", "-fopenmp", "-shared",
          "-fPIC"]


def build(force: bool = True) -> str:
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, os.path.join(_HERE, "orc.c"), "-lm"])
        os.replace(tmp, _SO)
    return _SO


class Cfg(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("input_mode", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("hidden", ctypes.c_int32), ("n_layers", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("max_ctx", ctypes.c_int32), ("n_seq", ctypes.c_int32), ("kv_f32", ctypes.c_int32),
                ("eps", ctypes.c_float), ("theta", ctypes.c_double)]


class Mat(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int32), ("cols", ctypes.c_int32), ("bf16", ctypes.c_void_p),
                ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("q8_0", ctypes.c_void_p)]


class Layer(ctypes.Structure):
    _fields_ = [("attn_norm", ctypes.c_void_p), ("q_norm", ctypes.c_void_p), ("k_norm", ctypes.c_void_p),
                ("mlp_norm", ctypes.c_void_p)] + [(n, Mat) for n in ("q", "k", "v", "o", "gate", "up", "down")]


_lib = None
_F = ctypes.c_void_p


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build(force=False)
        L = ctypes.CDLL(_SO)
        sig = {
            "orc_bf16_to_f32": (ctypes.c_float, [ctypes.c_uint16]),
            "orc_f32_to_bf16": (ctypes.c_uint16, [ctypes.c_float]),
            "orc_exp": (ctypes.c_float, [ctypes.c_float]),
            "orc_rmsnorm": (None, [_F, _F, ctypes.c_int32, ctypes.c_float, _F]),
            "orc_rope_table": (None, [ctypes.c_double, ctypes.c_int32, ctypes.c_int32, _F, _F]),
            "orc_rope_apply": (None, [_F, ctypes.c_int32, _F, _F]),
            "orc_softmax": (ctypes.c_int32, [_F, ctypes.c_int32, _F]),
            "orc_attention_head": (ctypes.c_int32, [_F, _F, _F, ctypes.c_int32, ctypes.c_int32, _F]),
            "orc_gqa_attention": (ctypes.c_int32, [_F, ctypes.c_int32, ctypes.c_int32, _F, _F, ctypes.c_size_t,
                                                   ctypes.c_int32, ctypes.c_int32, _F]),
            "orc_silu": (ctypes.c_float, [ctypes.c_float]),
            "orc_q8_dot": (ctypes.c_float, [_F, _F, _F, ctypes.c_int32]),
            "orc_q8_0_dot": (ctypes.c_float, [_F, _F, ctypes.c_int32]),
            "orc_f16_to_f32": (ctypes.c_float, [ctypes.c_uint16]),
            "orc_quantize_act8": (None, [_F, ctypes.c_int32, _F, _F]),
            "orc_q8q8_dot": (ctypes.c_float, [_F, _F, _F, _F, ctypes.c_int32]),
            "orc_bf16_dot": (ctypes.c_float, [_F, _F, ctypes.c_int32]),
            "orc_dequant_row": (None, [ctypes.POINTER(Mat), ctypes.c_int32, _F]),
            "orc_matvec": (None, [ctypes.POINTER(Mat), _F, _F]),
            "orc_argmax": (ctypes.c_int32, [_F, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)]),
            "orc_pcg32_seed": (None, [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p]),
            "orc_pcg32_next": (ctypes.c_uint32, [ctypes.c_void_p]),
            "orc_pcg32_uniform": (ctypes.c_float, [ctypes.c_uint32]),
            "orc_sample_prepare": (ctypes.c_int32, [_F, ctypes.c_int32, ctypes.c_float, _F, ctypes.c_int32, _F,
                                                    ctypes.c_int32, _F, _F]),
            "orc_sample": (ctypes.c_int32, [_F, ctypes.c_int32, ctypes.c_void_p, _F, ctypes.c_int32, _F,
                                            ctypes.c_int32, ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32), _F, _F,
                                            ctypes.POINTER(ctypes.c_int32)]),
            "orc_set_threads": (None, [ctypes.c_int32]),
            "orc_get_threads": (ctypes.c_int32, []),
            "orc_create": (ctypes.c_void_p, [ctypes.POINTER(Cfg), ctypes.POINTER(Mat), _F, ctypes.POINTER(Layer)]),
            "orc_destroy": (None, [ctypes.c_void_p]),
            "orc_step": (ctypes.c_int32, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, _F, _F, _F,
                                          ctypes.POINTER(ctypes.c_int32)]),
            "orc_step_kv": (ctypes.c_int32, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, _F, _F, _F,
                                             ctypes.POINTER(ctypes.c_int32), _F, _F]),
            "orc_kv_write": (ctypes.c_int32, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                              ctypes.c_int32, _F, _F]),
            "orc_kv_read": (ctypes.c_int32, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.c_int32, _F, _F]),
            "orc_set_len": (ctypes.c_int32, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32]),
            "orc_get_len": (ctypes.c_int32, [ctypes.c_void_p, ctypes.c_int32]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _p(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def f32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


# ---------------------------------------------------------------- building blocks (thin wrappers)
def rmsnorm(x, w, eps=1e-6):
    x, w = f32(x), f32(w)
    out = np.empty_like(x)
    lib().orc_rmsnorm(_p(x), _p(w), x.size, eps, _p(out))
    return out


def rope_table(theta, head_dim, pos):
    c = np.empty(head_dim // 2, np.float32)
    s = np.empty(head_dim // 2, np.float32)
    lib().orc_rope_table(theta, head_dim, pos, _p(c), _p(s))
    return c, s


def rope_apply(v, cos_t, sin_t):
    v = f32(v).copy()
    cos_t, sin_t = f32(cos_t), f32(sin_t)
    lib().orc_rope_apply(_p(v), v.size, _p(cos_t), _p(sin_t))
    return v


def softmax(s):
    s = f32(s)
    p = np.empty_like(s)
    rc = lib().orc_softmax(_p(s), s.size, _p(p))
    return rc, p


def attention_head(q, k_rows, v_rows):
    q, k_rows, v_rows = f32(q), f32(k_rows), f32(v_rows)
    out = np.empty(q.size, np.float32)
    rc = lib().orc_attention_head(_p(q), _p(k_rows), _p(v_rows), k_rows.shape[0], q.size, _p(out))
    return rc, out


def gqa_attention(q, k_heads, v_heads):
    """q [n_q, D]; k_heads, v_heads [n_kv, n, D] -> (rc, out [n_q, D])."""
    q, k_heads, v_heads = f32(q), f32(k_heads), f32(v_heads)
    n_q, D = q.shape
    n_kv, n, _ = k_heads.shape
    out = np.empty((n_q, D), np.float32)
    rc = lib().orc_gqa_attention(_p(q), n_q, n_kv, _p(k_heads), _p(v_heads), n * D, n, D, _p(out))
    return rc, out


def silu(z):
    return np.float32(lib().orc_silu(float(np.float32(z))))


def q8_dot(codes, scales, act):
    codes = np.ascontiguousarray(codes, np.int8)
    scales, act = f32(scales), f32(act)
    return np.float32(lib().orc_q8_dot(_p(codes), _p(scales), _p(act), codes.size))


def q8_0_dot(blocks, act):
    """blocks: uint8 [n/32 * 34] (little-endian f16 scale, 32 int8 codes per block)."""
    blocks = np.ascontiguousarray(blocks, np.uint8)
    act = f32(act)
    return np.float32(lib().orc_q8_0_dot(_p(blocks), _p(act), act.size))


def quantize_act8(x):
    """Per-32-block int8 codes and f32 scales of an activation vector."""
    x = f32(x)
    q = np.empty(x.size, np.int8)
    d = np.empty(x.size // 32, np.float32)
    lib().orc_quantize_act8(_p(x), x.size, _p(q), _p(d))
    return q, d


def q8q8_dot(codes, scales, aq, ad):
    codes = np.ascontiguousarray(codes, np.int8)
    aq = np.ascontiguousarray(aq, np.int8)
    return np.float32(lib().orc_q8q8_dot(_p(codes), _p(f32(scales)), _p(aq), _p(f32(ad)), codes.size))


def f16_to_f32(bits):
    return np.float32(lib().orc_f16_to_f32(int(bits)))


def bf16_dot(w_bits, act):
    w_bits = np.ascontiguousarray(w_bits, np.uint16)
    act = f32(act)
    return np.float32(lib().orc_bf16_dot(_p(w_bits), _p(act), w_bits.size))


def argmax(v):
    v = f32(v)
    idx = ctypes.c_int32(-1)
    rc = lib().orc_argmax(_p(v), v.size, ctypes.byref(idx))
    return rc, idx.value


class Pcg32(ctypes.Structure):
    """PCG32 generator state (state, odd increment) of the sampling contract."""
    _fields_ = [("state", ctypes.c_uint64), ("inc", ctypes.c_uint64)]

    @classmethod
    def seeded(cls, seed, stream_id):
        r = cls()
        lib().orc_pcg32_seed(seed, stream_id, ctypes.byref(r))
        return r

    def next(self):
        return int(lib().orc_pcg32_next(ctypes.byref(self)))


def pcg32_uniform(word):
    return float(lib().orc_pcg32_uniform(int(word)))


class SampleParams(ctypes.Structure):
    _fields_ = [("temperature", ctypes.c_float), ("top_p", ctypes.c_float), ("repetition_penalty", ctypes.c_float),
                ("top_k", ctypes.c_int32)]


def _i32(a):
    return np.ascontiguousarray(np.asarray(a if a is not None else [], np.int32))


def sample_prepare(logits, penalty=1.0, history=None, forbid=None):
    """Steps 1-5 of the sampling order: (rc, transformed logits)."""
    lg = f32(logits)
    h, fb = _i32(history), _i32(forbid)
    z = np.empty_like(lg)
    seen = np.zeros(lg.size, np.uint8)
    rc = lib().orc_sample_prepare(_p(lg), lg.size, penalty, _p(h) if h.size else None, h.size,
                                  _p(fb) if fb.size else None, fb.size, _p(z), _p(seen))
    return rc, z


def sample(logits, rng, temperature=1.0, top_k=50, top_p=1.0, penalty=1.0, history=None, forbid=None):
    """One draw; returns (rc, token, candidate ids in draw order, their final probabilities).  `rng` (Pcg32) is
    advanced in place (not at temperature 0)."""
    lg = f32(logits)
    h, fb = _i32(history), _i32(forbid)
    prm = SampleParams(temperature, top_p, penalty, top_k)
    tok = ctypes.c_int32(-1)
    n = ctypes.c_int32(0)
    probs = np.empty(lg.size, np.float32)
    ids = np.empty(lg.size, np.int32)
    rc = lib().orc_sample(_p(lg), lg.size, ctypes.byref(prm), _p(h) if h.size else None, h.size,
                          _p(fb) if fb.size else None, fb.size, ctypes.byref(rng) if rng is not None else None,
                          ctypes.byref(tok), _p(probs), _p(ids), ctypes.byref(n))
    return rc, tok.value, ids[:n.value].copy(), probs[:n.value].copy()


def set_threads(n):
    lib().orc_set_threads(int(n))


def get_threads():
    return lib().orc_get_threads()


def mat_struct(m) -> Mat:
    """m: synth.Matrix (bf16 bits, int8 codes + f32 scales, or Q8_0 34-byte blocks, which take precedence)."""
    if getattr(m, "q8_0", None) is not None:
        return Mat(m.rows, m.cols, None, None, None, _p(m.q8_0))
    if m.is_q8:
        return Mat(m.rows, m.cols, None, _p(m.codes), _p(m.scales), None)
    return Mat(m.rows, m.cols, _p(m.bf16), None, None, None)


def dequant_row(m, row):
    out = np.empty(m.cols, np.float32)
    ms = mat_struct(m)
    lib().orc_dequant_row(ctypes.byref(ms), row, _p(out))
    return out


def matvec(m, x):
    x = f32(x)
    out = np.empty(m.rows, np.float32)
    ms = mat_struct(m)
    lib().orc_matvec(ctypes.byref(ms), _p(x), _p(out))
    return out


class Model:
    """Whole-model oracle over a ``synth.Weights`` (arrays are borrowed; keep ``weights`` alive)."""

    def __init__(self, weights, n_seq=None, max_ctx=None, kv_f32=False):
        s = weights.shape
        self.weights = weights
        self.shape = s
        self.n_seq = n_seq or s.n_seq
        self.max_ctx = max_ctx or s.max_ctx
        self.cfg = Cfg(s.fmt, s.input_mode, s.vocab, s.hidden, s.n_layers, s.n_q_heads, s.n_kv_heads, s.head_dim,
                       s.inter, self.max_ctx, self.n_seq, 1 if kv_f32 else 0, s.eps, s.theta)
        layers = (Layer * s.n_layers)()
        for l, d in enumerate(weights.layers):
            layers[l].attn_norm = _p(d["attn_norm"])
            layers[l].q_norm = _p(d["q_norm"])
            layers[l].k_norm = _p(d["k_norm"])
            layers[l].mlp_norm = _p(d["mlp_norm"])
            for n in ("q", "k", "v", "o", "gate", "up", "down"):
                setattr(layers[l], n, mat_struct(d[n]))
        self._layers = layers
        self._embed = mat_struct(weights.embed) if weights.embed is not None else None
        fn = _p(weights.final_norm) if weights.final_norm is not None else None
        h = lib().orc_create(ctypes.byref(self.cfg), ctypes.byref(self._embed) if self._embed else None, fn, layers)
        if not h:
            raise ValueError("oracle rejected the model shape")
        self.h = h

    def close(self):
        if getattr(self, "h", None) and _lib is not None:
            _lib.orc_destroy(self.h)
        self.h = None

    def __del__(self):
        self.close()

    def step(self, seq=0, tok=-1, hidden_in=None, want_logits=True, want_hidden=False, want_argmax=True):
        """Returns (rc, argmax, logits or None, hidden_out or None).  With neither logits nor argmax
        requested the final norm and logits are skipped (a prefill position that is not the last)."""
        hin = f32(hidden_in) if hidden_in is not None else None
        hout = np.empty(self.shape.hidden, np.float32) if want_hidden else None
        lg = np.empty(self.shape.vocab, np.float32) if (want_logits and self.shape.input_mode == 0) else None
        am = ctypes.c_int32(-1)
        rc = lib().orc_step(self.h, seq, int(tok), _p(hin), _p(hout), _p(lg),
                            ctypes.byref(am) if (self.shape.input_mode == 0 and want_argmax) else None)
        return rc, am.value, lg, hout

    def step_forced(self, seq, tok=-1, kv_force=None, hidden_in=None, want_hidden=False):
        """A step whose appended position takes the given bf16 K/V bits (uint16 [L][2][HKV][D]: K heads then V
        heads per layer) instead of the oracle's own rounding.  Returns (rc, argmax, logits or None, hidden or
        None, own) where own holds the oracle's own bf16 K/V bits of that position in the same layout."""
        s = self.shape
        hin = f32(hidden_in) if hidden_in is not None else None
        hout = np.empty(s.hidden, np.float32) if want_hidden else None
        lg = np.empty(s.vocab, np.float32) if s.input_mode == 0 else None
        own = np.empty((s.n_layers, 2, s.n_kv_heads, s.head_dim), np.uint16)
        force = None if kv_force is None else np.ascontiguousarray(kv_force, np.uint16)
        am = ctypes.c_int32(-1)
        rc = lib().orc_step_kv(self.h, seq, int(tok), _p(hin), _p(hout), _p(lg),
                               ctypes.byref(am) if s.input_mode == 0 else None, _p(force), _p(own))
        return rc, am.value, lg, hout, own

    def prefill(self, tokens, seq=0):
        """Token-by-token prefill; returns (rc, argmax, logits) of the last position."""
        rc, am, lg = ORC_OK, -1, None
        for i, t in enumerate(tokens):
            last = i == len(tokens) - 1
            rc, am, lg, _ = self.step(seq, int(t), want_logits=last, want_argmax=last)
            if rc != ORC_OK:
                break
        return rc, am, lg

    def kv_write(self, seq, layer, pos0, k_bits, v_bits):
        k_bits = np.ascontiguousarray(k_bits, np.uint16)
        v_bits = np.ascontiguousarray(v_bits, np.uint16)
        n_pos = k_bits.shape[1]
        return lib().orc_kv_write(self.h, seq, layer, pos0, n_pos, _p(k_bits), _p(v_bits))

    def kv_read(self, seq, layer, pos0, n_pos):
        s = self.shape
        k = np.empty((s.n_kv_heads, n_pos, s.head_dim), np.uint16)
        v = np.empty_like(k)
        rc = lib().orc_kv_read(self.h, seq, layer, pos0, n_pos, _p(k), _p(v))
        return rc, k, v

    def set_len(self, seq, n):
        return lib().orc_set_len(self.h, seq, n)

    def get_len(self, seq):
        return lib().orc_get_len(self.h, seq)
