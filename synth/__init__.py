"""Seeded synthetic inputs for the Qwen3-0.6B-shaped decoder.

Test and benchmark infrastructure used by both the oracle side and the GPU
side of every parity check.  It only draws random numbers (PCG32 streams, see
``synth.c``) and rounds them to storage types; none of the decoder's
arithmetic lives here.

Tensor inventory and canonical order follow "M1 — Load the weights", section
"What it prints" (the per-block tensor table): embed_tokens, then per block
input_layernorm, q_proj, k_proj, v_proj, q_norm, k_norm, o_proj,
post_attention_layernorm, gate_proj, up_proj, down_proj, then model.norm.
Matrices are stored [out, in] row-major (y = x W^T).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")

SYN_NORMAL_F32, SYN_NORMAL_BF16, SYN_UNIFORM_F32, SYN_INT8, SYN_INT32 = range(5)

FMT_BF16 = 1
FMT_Q8 = 2
FMT_Q8_0 = 3     # Q8 with the pages' block layout: per 32 codes a 34-byte block led by a little-endian f16 scale
FMT_Q8_ACT8 = 4  # Q8 weights (codes + f32 scales) whose products quantize the activations to int8 on the fly
INPUT_TOKENS = 0
INPUT_HIDDEN = 1

# per-block tensor slots, canonical order
LAYER_SLOTS = ("attn_norm", "q", "k", "v", "q_norm", "k_norm", "o", "mlp_norm", "gate", "up", "down")
MATRIX_SLOTS = ("q", "k", "v", "o", "gate", "up", "down")


def build(force: bool = True) -> str:
    src = os.path.join(_HERE, "synth.c")
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-o", tmp, src, "-lm"])
        os.replace(tmp, _SO)
    return _SO


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build(force=False)
        L = ctypes.CDLL(_SO)
        L.syn_fill.argtypes = [ctypes.c_int, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_double,
                               ctypes.c_double, ctypes.c_void_p]
        L.syn_fill.restype = ctypes.c_uint32
        L.syn_pcg32_words.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p]
        L.syn_pcg32_words.restype = ctypes.c_uint32
        _lib = L
    return _lib


def pcg32_words(seed: int, stream_id: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.uint32)
    lib().syn_pcg32_words(seed, stream_id, n, out.ctypes.data)
    return out


def _fill(kind, dtype, seed, tid, shape, a, b):
    out = np.empty(shape, dtype=dtype)
    n = int(np.prod(shape))
    if n:
        rc = lib().syn_fill(kind, seed, tid, n, float(a), float(b), out.ctypes.data)
        assert rc == 0
    return out


def normal_f32(seed, tid, shape, mean=0.0, std=1.0):
    return _fill(SYN_NORMAL_F32, np.float32, seed, tid, shape, mean, std)


def normal_bf16(seed, tid, shape, mean=0.0, std=1.0):
    """bf16 bit patterns (uint16), rounded to nearest even from the f32 draw."""
    return _fill(SYN_NORMAL_BF16, np.uint16, seed, tid, shape, mean, std)


def uniform_f32(seed, tid, shape, lo, hi):
    return _fill(SYN_UNIFORM_F32, np.float32, seed, tid, shape, lo, hi)


def int8_uniform(seed, tid, shape, lo=-127, hi=127):
    return _fill(SYN_INT8, np.int8, seed, tid, shape, lo, hi)


def int32_uniform(seed, tid, shape, lo, hi):
    return _fill(SYN_INT32, np.int32, seed, tid, shape, lo, hi)


def bf16_to_f32(u16: np.ndarray) -> np.ndarray:
    return (u16.astype(np.uint32) << 16).view(np.float32)


@dataclass(frozen=True)
class ModelShape:
    """Every dimension explicit; nothing defaulted from tensor names."""
    fmt: int = FMT_BF16
    input_mode: int = INPUT_TOKENS
    vocab: int = 151936
    hidden: int = 1024
    n_layers: int = 28
    n_q_heads: int = 16
    n_kv_heads: int = 8
    head_dim: int = 128
    inter: int = 3072
    max_ctx: int = 4096
    n_seq: int = 1
    eps: float = 1e-6
    theta: float = 1e6
    max_prefill: int = 2048

    @property
    def q_dim(self):
        return self.n_q_heads * self.head_dim

    @property
    def kv_dim(self):
        return self.n_kv_heads * self.head_dim

    def matrix_shape(self, slot):
        H, Q, KV, I = self.hidden, self.q_dim, self.kv_dim, self.inter
        return {"q": (Q, H), "k": (KV, H), "v": (KV, H), "o": (H, Q), "gate": (I, H), "up": (I, H),
                "down": (H, I)}[slot]

    def norm_len(self, slot):
        return {"attn_norm": self.hidden, "mlp_norm": self.hidden, "q_norm": self.head_dim,
                "k_norm": self.head_dim}[slot]


# Qwen3-0.6B dimensions ("M1 — Load the weights", dimensions table)
QWEN3_06B = ModelShape()


def tensor_id(slot: str, layer: int, n_layers: int) -> int:
    if slot == "embed":
        return 0
    if slot == "final_norm":
        return 1 + 11 * n_layers
    return 1 + 11 * layer + LAYER_SLOTS.index(slot)


SCALE_ID = 1 << 20       # offset of a Q8 matrix's scale stream
TOKENS_ID = 1 << 24      # token-id streams
HIDDEN_ID = 1 << 25      # fp32 hidden-state inputs
KV_ID = 1 << 26          # KV-cache fill streams
LOGITS_ID = 1 << 27      # synthetic logits rows (sampling inputs)


@dataclass
class Matrix:
    """Canonical [rows, cols] matrix: bf16 bits, or Q8 int8 codes + f32 scales [rows, cols/32].  For the
    Q8_0 format also the 34-byte blocks [rows, cols/32 * 34] (f16 scale bits little-endian, then the 32
    codes); its `scales` then hold the f16 scale values widened to f32 (exact)."""
    rows: int
    cols: int
    bf16: np.ndarray | None = None
    codes: np.ndarray | None = None
    scales: np.ndarray | None = None
    q8_0: np.ndarray | None = None

    @property
    def is_q8(self):
        return self.codes is not None


@dataclass
class Weights:
    shape: ModelShape
    embed: Matrix | None
    final_norm: np.ndarray | None       # bf16 bits (FMT_BF16) or f32 (FMT_Q8)
    layers: list = field(default_factory=list)  # dict slot -> Matrix | ndarray


def _matrix(shape: ModelShape, seed: int, tid: int, rows: int, cols: int, std: float) -> Matrix:
    if shape.fmt == FMT_BF16:
        return Matrix(rows, cols, bf16=normal_bf16(seed, tid, (rows, cols), 0.0, std))
    assert cols % 32 == 0
    codes = int8_uniform(seed, tid, (rows, cols), -127, 127)
    scales = uniform_f32(seed, tid + SCALE_ID, (rows, cols // 32), 1e-3, 1e-2)
    if shape.fmt in (FMT_Q8, FMT_Q8_ACT8):
        return Matrix(rows, cols, codes=codes, scales=scales)
    return q8_0_matrix(codes, scales.astype(np.float16))


def q8_0_matrix(codes: np.ndarray, scales16: np.ndarray) -> Matrix:
    """Packs int8 codes [rows, cols] and f16 scales [rows, cols/32] into Q8_0 blocks."""
    rows, cols = codes.shape
    nb = cols // 32
    blk = np.empty((rows, nb, 34), np.uint8)
    blk[:, :, :2] = np.ascontiguousarray(scales16.astype("<f2")).view(np.uint8).reshape(rows, nb, 2)
    blk[:, :, 2:] = codes.reshape(rows, nb, 32).view(np.uint8)
    return Matrix(rows, cols, codes=codes, scales=scales16.astype(np.float32), q8_0=blk.reshape(rows, nb * 34))


def _norm(shape: ModelShape, seed: int, tid: int, n: int):
    if shape.fmt == FMT_BF16:
        return normal_bf16(seed, tid, (n,), 1.0, 0.1)
    return normal_f32(seed, tid, (n,), 1.0, 0.1)


def make_weights(shape: ModelShape, seed: int, w_std: float = 0.02) -> Weights:
    """bf16: matrices ~N(0, w_std) and norms 1+N(0,0.1), rounded to bf16.
    Q8: codes uniform in [-127,127], scales ~U(1e-3,1e-2), norms f32 1+N(0,0.1)."""
    L = shape.n_layers
    embed = final = None
    if shape.input_mode == INPUT_TOKENS:
        embed = _matrix(shape, seed, tensor_id("embed", 0, L), shape.vocab, shape.hidden, w_std)
        final = _norm(shape, seed, tensor_id("final_norm", 0, L), shape.hidden)
    layers = []
    for l in range(L):
        d = {}
        for slot in LAYER_SLOTS:
            tid = tensor_id(slot, l, L)
            if slot in MATRIX_SLOTS:
                r, c = shape.matrix_shape(slot)
                d[slot] = _matrix(shape, seed, tid, r, c, w_std)
            else:
                d[slot] = _norm(shape, seed, tid, shape.norm_len(slot))
        layers.append(d)
    return Weights(shape, embed, final, layers)


def tokens(seed: int, purpose: int, n: int, vocab: int) -> np.ndarray:
    return int32_uniform(seed, TOKENS_ID + purpose, (n,), 0, vocab - 1)


def hidden_inputs(seed: int, purpose: int, n: int, hidden: int) -> np.ndarray:
    return normal_f32(seed, HIDDEN_ID + purpose, (n, hidden), 0.0, 1.0)


def logits_rows(seed: int, purpose: int, rows: int, vocab: int, std: float = 3.0) -> np.ndarray:
    """f32 N(0, std) rows standing in for a decode step's logits (the Q8 workload's logits have RMS ~14, the
    bf16 workload's ~1-3)."""
    return normal_f32(seed, LOGITS_ID + purpose, (rows, vocab), 0.0, std)


def kv_fill(seed: int, seq: int, layer: int, n_kv: int, n_pos: int, head_dim: int):
    """bf16 N(0,1) K and V for one (sequence, layer): arrays [n_kv, n_pos, head_dim] of bf16 bits."""
    base = KV_ID + (seq * 4096 + layer) * 2
    k = normal_bf16(seed, base, (n_kv, n_pos, head_dim))
    v = normal_bf16(seed, base + 1, (n_kv, n_pos, head_dim))
    return k, v


# ---------------------------------------------------------------------------------------------
# The five workloads (shapes, seeds and input recipe)
# ---------------------------------------------------------------------------------------------
@dataclass(frozen=True)
class Workload:
    name: str
    shape: ModelShape
    seed: int
    prefill: int = 0          # tokens prefilled by the prefill entry point
    decode: int = 0           # greedy decode steps
    kv_prefill: int = 0       # positions filled synthetically via kv_write
    hidden_decode: int = 0    # fp32 hidden vectors fed one per step (single-block workload)


SINGLE_BLOCK = Workload("single-block bf16: prefill 16 + decode 16 hidden states",
                        replace(QWEN3_06B, n_layers=1, input_mode=INPUT_HIDDEN, vocab=0, max_ctx=64,
                                max_prefill=64), seed=1, prefill=16, hidden_decode=16)
BF16_DECODE = Workload("28-layer bf16 B=1: prefill 128 + 256 greedy decode",
                       replace(QWEN3_06B, max_ctx=512, max_prefill=128), seed=2, prefill=128, decode=256)
Q8_DECODE = Workload("28-layer Q8 B=1 decode at KV context 2048",
                     replace(QWEN3_06B, fmt=FMT_Q8, max_ctx=2048 + 512, max_prefill=16), seed=3, kv_prefill=2048,
                     decode=128)
BF16_PREFILL = Workload("28-layer bf16 B=1 prefill 2048",
                        replace(QWEN3_06B, max_ctx=2048, max_prefill=2048), seed=4, prefill=2048)
Q8_BATCHED = Workload("28-layer Q8 16 sequences x KV context 8192, 64 greedy iterations",
                      replace(QWEN3_06B, fmt=FMT_Q8, max_ctx=8192 + 64, n_seq=16, max_prefill=16), seed=5,
                      kv_prefill=8192, decode=64)

WORKLOADS = (SINGLE_BLOCK, BF16_DECODE, Q8_DECODE, BF16_PREFILL, Q8_BATCHED)


# ---------------------------------------------------------------------------------------------
# Marshalling helpers: the canonical tensors and shape as plain dicts for the library binding
# ---------------------------------------------------------------------------------------------
def abi_config_kwargs(shape: ModelShape) -> dict:
    return dict(weight_format=shape.fmt, input_mode=shape.input_mode, vocab=shape.vocab, hidden=shape.hidden,
                n_layers=shape.n_layers, n_q_heads=shape.n_q_heads, n_kv_heads=shape.n_kv_heads,
                head_dim=shape.head_dim, inter=shape.inter, max_ctx=shape.max_ctx, n_seq=shape.n_seq,
                max_prefill=shape.max_prefill, eps=shape.eps, theta=shape.theta)


def abi_tensors(w: Weights, with_lm_head: bool = False) -> list:
    """Tensor list (kind name, layer, dtype code, arrays) in the order of the inventory; dtype codes
    1 = bf16 bits, 2 = f32, 3 = int8 codes + f32 scales, 4 = Q8_0 34-byte blocks."""
    q8 = w.shape.fmt in (FMT_Q8, FMT_Q8_0, FMT_Q8_ACT8)
    out = []

    def mat(kind, layer, m):
        if w.shape.fmt == FMT_Q8_0:
            out.append(dict(kind=kind, layer=layer, dtype=4, data=m.q8_0))
        elif q8:
            out.append(dict(kind=kind, layer=layer, dtype=3, data=m.codes, scales=m.scales))
        else:
            out.append(dict(kind=kind, layer=layer, dtype=1, data=m.bf16))

    def vec(kind, layer, v):
        out.append(dict(kind=kind, layer=layer, dtype=2 if q8 else 1, data=v))

    if w.embed is not None:
        mat("embed", -1, w.embed)
        vec("final_norm", -1, w.final_norm)
        if with_lm_head:
            mat("lm_head", -1, w.embed)
    for l, d in enumerate(w.layers):
        for slot in LAYER_SLOTS:
            if slot in MATRIX_SLOTS:
                mat(slot, l, d[slot])
            else:
                vec(slot, l, d[slot])
    return out
