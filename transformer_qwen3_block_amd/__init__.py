"""Python binding of libqw3, the gfx950 Qwen3 decoder-block library (C ABI in include/qw3.h).

Argument marshalling only: every step of the forward pass runs in the library's HIP kernels.  PyTorch is
used for device memory (the arena and the caller's input/output tensors) and for the current HIP stream.
Importing works without a GPU (host-side validation can be exercised); calls that need the device raise
if the native library is missing -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(_HERE)
_SO = os.path.join(_HERE, "libqw3.so")
_SOURCES = ["api.hip", "decode.hip", "prefill.hip", "mega.hip", "gemv_mfma.hip", "sample.hip", "loader.cpp",
            "probe.hip"]

ABI_VERSION = 1
WEIGHTS_BF16, WEIGHTS_Q8, WEIGHTS_Q8_0, WEIGHTS_Q8_ACT8 = 1, 2, 3, 4
INPUT_TOKENS, INPUT_HIDDEN = 0, 1
DT_BF16, DT_F32, DT_Q8, DT_Q8_0 = 1, 2, 3, 4
KIND = {"embed": 0, "final_norm": 1, "lm_head": 2, "attn_norm": 3, "q": 4, "k": 5, "v": 6, "q_norm": 7,
        "k_norm": 8, "o": 9, "mlp_norm": 10, "gate": 11, "up": 12, "down": 13}
STATUS = {0: "Ok", 1: "InvalidArgument", 2: "UnsupportedAbi", 4: "InvalidHandle", 5: "StaleHandle", 6: "Bounds",
          7: "Alignment", 8: "IntegerOverflow", 9: "OutOfMemory", 10: "InvalidModel", 12: "UnsupportedQuantization",
          13: "UnsupportedShape", 14: "ContextExceeded", 18: "NumericalFailure", 20: "InternalInvariant",
          21: "DeviceError"}

HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
               # no packed-FP32 instructions in device code
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


class Qw3Error(RuntimeError):
    def __init__(self, code, what):
        super().__init__(f"{what}: {STATUS.get(code, code)} ({code})")
        self.code = code


def build(force: bool = True) -> str:
    """Compile libqw3.so for gfx950 in-tree."""
    if force or not os.path.exists(_SO):
        hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
        srcs = [os.path.join(_HERE, "csrc", s) for s in _SOURCES]
        tmp = _SO + ".tmp"
        cmd = [hipcc, *HIPCC_FLAGS, "-I", os.path.join(_ROOT, "include"), "-I", os.path.join(_HERE, "csrc"), *srcs,
               "-o", tmp]
        subprocess.check_call(cmd)
        os.replace(tmp, _SO)
    return _SO


class Config(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_uint32), ("weight_format", ctypes.c_uint32), ("input_mode", ctypes.c_uint32),
                ("vocab_size", ctypes.c_int32), ("hidden", ctypes.c_int32), ("n_layers", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("intermediate", ctypes.c_int32), ("max_ctx", ctypes.c_int32), ("n_seq", ctypes.c_int32),
                ("max_prefill", ctypes.c_int32), ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_double)]


class Sizes(ctypes.Structure):
    _fields_ = [("total", ctypes.c_uint64), ("weights", ctypes.c_uint64), ("kv", ctypes.c_uint64),
                ("scratch", ctypes.c_uint64), ("state", ctypes.c_uint64)]


class Tensor(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("layer", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("data", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


EXPORTS = ["qw3_abi_version", "qw3_rope_table", "qw3_preflight", "qw3_create", "qw3_load_weights", "qw3_prefill", "qw3_decode_step",
           "qw3_reset_kv", "qw3_status_poll", "qw3_get_len", "qw3_destroy", "qw3_block_forward", "qw3_kv_write",
           "qw3_kv_read", "qw3_kv_set_len", "qw3_dequant", "qw3_bench_kernel", "qw3_pcg32_seed",
           "qw3_sample_workspace_bytes", "qw3_sample", "qw3_inspect_file", "qw3_load_file",
           "qw3_sample_noalloc", "qw3_probe_hbm_read", "qw3_probe_mfma_f16"]

_lib = None


def lib():
    """Load libqw3.so (built by build()); raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            raise RuntimeError(f"native library {_SO} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(_SO)
        V, I32, U64, P = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64, ctypes.c_void_p
        sig = {
            "qw3_abi_version": (ctypes.c_uint32, []),
            "qw3_rope_table": (I32, [ctypes.c_double, I32, I32, P, P]),
            "qw3_preflight": (I32, [ctypes.POINTER(Config), ctypes.POINTER(Sizes)]),
            "qw3_create": (I32, [ctypes.POINTER(Config), V, U64, ctypes.POINTER(U64)]),
            "qw3_load_weights": (I32, [U64, ctypes.POINTER(Tensor), I32, V]),
            "qw3_prefill": (I32, [U64, I32, P, I32, P, P, V]),
            "qw3_decode_step": (I32, [U64, P, P, P, V]),
            "qw3_reset_kv": (I32, [U64, I32]),
            "qw3_status_poll": (I32, [U64, V]),
            "qw3_get_len": (I32, [U64, I32, ctypes.POINTER(I32)]),
            "qw3_destroy": (I32, [U64]),
            "qw3_block_forward": (I32, [U64, P, I32, P, V]),
            "qw3_kv_write": (I32, [U64, I32, I32, I32, I32, P, P, V]),
            "qw3_kv_read": (I32, [U64, I32, I32, I32, I32, P, P, V]),
            "qw3_kv_set_len": (I32, [U64, I32, I32, V]),
            "qw3_dequant": (I32, [U64, I32, I32, P, V]),
            "qw3_bench_kernel": (I32, [U64, I32, I32, I32, V]),
            "qw3_pcg32_seed": (I32, [U64, U64, P]),
            "qw3_sample_noalloc": (I32, [P, I32, I32, ctypes.c_int64, ctypes.POINTER(SampleParams), P, I32, P, I32,
                                         P, I32, P, P, P, P, V]),
            "qw3_probe_hbm_read": (I32, [P, U64, P, I32, V]),
            "qw3_probe_mfma_f16": (I32, [I32, I32, P, V]),
            "qw3_inspect_file": (I32, [ctypes.c_char_p, ctypes.POINTER(FileReport)]),
            "qw3_load_file": (I32, [U64, ctypes.c_char_p, V]),
            "qw3_sample_workspace_bytes": (I32, [I32, ctypes.POINTER(U64)]),
            "qw3_sample": (I32, [P, I32, I32, ctypes.c_int64, ctypes.POINTER(SampleParams), P, I32, P, I32, P, I32,
                                 P, P, P, P, P, U64, V]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


class FileReport(ctypes.Structure):
    _fields_ = [("n_tensors", ctypes.c_int64), ("stored_params", ctypes.c_int64), ("logical_params", ctypes.c_int64),
                ("embed_params", ctypes.c_int64), ("header_bytes", ctypes.c_int64), ("n_layers", ctypes.c_int32),
                ("lm_head_present", ctypes.c_int32)]


def inspect_file(path):
    """Validates a safetensors / SLM2 weight file on the host (no device); returns its FileReport."""
    r = FileReport()
    check(lib().qw3_inspect_file(os.fsencode(path), ctypes.byref(r)), "qw3_inspect_file")
    return r


class SampleParams(ctypes.Structure):
    _fields_ = [("temperature", ctypes.c_float), ("top_p", ctypes.c_float), ("repetition_penalty", ctypes.c_float),
                ("top_k", ctypes.c_int32)]


def pcg32_seed(seed, stream_id):
    """(state, increment) of the sampling generator for (seed, stream_id)."""
    out = (ctypes.c_uint64 * 2)()
    check(lib().qw3_pcg32_seed(seed, stream_id, out), "qw3_pcg32_seed")
    return int(out[0]), int(out[1])


class Sampler:
    """Deterministic sampling of token ids from device logits rows (qw3_sample); owns its device workspace and
    one PCG32 generator per row."""

    def __init__(self, n_rows, seeds, stream_ids=None, device="cuda:0"):
        import torch
        self.n_rows = n_rows
        self.device = torch.device(device)
        nb = ctypes.c_uint64(0)
        check(lib().qw3_sample_workspace_bytes(n_rows, ctypes.byref(nb)), "qw3_sample_workspace_bytes")
        self._ws = torch.empty(int(nb.value) + 256, dtype=torch.uint8, device=self.device)
        self._ws_ptr = (self._ws.data_ptr() + 255) & ~255
        self._ws_bytes = int(nb.value)
        sids = stream_ids if stream_ids is not None else list(range(n_rows))
        st = [pcg32_seed(int(seeds[r]), int(sids[r])) for r in range(n_rows)]
        self.rng = torch.tensor(np.array(st, np.uint64).view(np.int64), device=self.device)

    def __call__(self, logits, temperature=1.0, top_k=50, top_p=1.0, penalty=1.0, history=None, forbid=None,
                 stop=(), stream=None, status=None, done=None):
        """logits: f32 [n_rows, ld] device tensor (the first `vocab` = logits.shape[1] columns); history int32
        [n_rows, n] device tensor or None; forbid int32 [m] device tensor or None.  Returns token ids (int32
        [n_rows] device tensor)."""
        import torch
        tok = torch.empty(self.n_rows, dtype=torch.int32, device=self.device)
        prm = SampleParams(temperature, top_p, penalty, top_k)
        stop_arr = (ctypes.c_int32 * max(1, len(stop)))(*stop)
        nh = 0 if history is None else history.shape[1]
        nf = 0 if forbid is None else forbid.numel()
        check(lib().qw3_sample(_ptr(logits), self.n_rows, logits.shape[1], logits.stride(0), ctypes.byref(prm),
                               _ptr(history), nh, _ptr(forbid), nf, stop_arr if stop else None, len(stop),
                               _ptr(self.rng), _ptr(tok), _ptr(done), _ptr(status), ctypes.c_void_p(self._ws_ptr),
                               self._ws_bytes, _stream(stream)), "qw3_sample")
        return tok


def check(rc, what):
    if rc != 0:
        raise Qw3Error(rc, what)


def make_config(*, weight_format, input_mode, vocab, hidden, n_layers, n_q_heads, n_kv_heads, head_dim, inter,
                max_ctx, n_seq, max_prefill, eps, theta, abi_version=ABI_VERSION) -> Config:
    return Config(abi_version, weight_format, input_mode, vocab, hidden, n_layers, n_q_heads, n_kv_heads, head_dim,
                  inter, max_ctx, n_seq, max_prefill, eps, theta)


def preflight(cfg: Config) -> Sizes:
    sz = Sizes()
    check(lib().qw3_preflight(ctypes.byref(cfg), ctypes.byref(sz)), "qw3_preflight")
    return sz


def rope_table(theta, head_dim, n_pos):
    """The library's host-built RoPE table: (cos, sin) f32 [n_pos, head_dim/2]."""
    c = np.empty((n_pos, head_dim // 2), np.float32)
    s = np.empty((n_pos, head_dim // 2), np.float32)
    check(lib().qw3_rope_table(theta, head_dim, n_pos, c.ctypes.data, s.ctypes.data), "qw3_rope_table")
    return c, s


def _ptr(t):
    """Device pointer of a torch tensor (or None)."""
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _np_ptr(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


class Model:
    """One model instance in a device arena allocated through torch."""

    def __init__(self, cfg: Config, device="cuda:0"):
        import torch
        self.cfg = cfg
        self.device = torch.device(device)
        self.sizes = preflight(cfg)
        # 256-byte aligned arena (torch's caching allocator returns >= 512-byte aligned blocks)
        self.arena = torch.empty(int(self.sizes.total) + 256, dtype=torch.uint8, device=self.device)
        base = self.arena.data_ptr()
        self._base = (base + 255) & ~255
        h = ctypes.c_uint64(0)
        check(lib().qw3_create(ctypes.byref(cfg), ctypes.c_void_p(self._base), self.sizes.total, ctypes.byref(h)),
              "qw3_create")
        self.handle = h.value

    # -------------------------------------------------------------------------------- weights
    def load_weights(self, tensors, stream=None):
        """tensors: list of dicts {kind, layer, dtype, data (np array), scales (np array or None)}."""
        arr = (Tensor * len(tensors))()
        keep = []
        for i, t in enumerate(tensors):
            data = np.ascontiguousarray(t["data"])
            sc = None if t.get("scales") is None else np.ascontiguousarray(t["scales"], dtype=np.float32)
            keep += [data, sc]
            rows, cols = (1, data.shape[0]) if data.ndim == 1 else data.shape
            if t["dtype"] == DT_Q8_0:   # [rows, blocks * 34] bytes -> [rows, blocks * 32] inputs
                cols = cols // 34 * 32
            arr[i] = Tensor(KIND[t["kind"]] if isinstance(t["kind"], str) else t["kind"], t.get("layer", -1),
                            t["dtype"], 0, rows, cols, data.ctypes.data, sc.ctypes.data if sc is not None else None)
        check(lib().qw3_load_weights(self.handle, arr, len(tensors), _stream(stream)), "qw3_load_weights")

    def load_file(self, path, stream=None):
        """Weights from a safetensors (bf16) or SLM2 (Q8_0 blocks + f32 norms) file."""
        check(lib().qw3_load_file(self.handle, os.fsencode(path), _stream(stream)), "qw3_load_file")

    # -------------------------------------------------------------------------------- forward
    def prefill(self, tokens, seq=0, logits=None, argmax=None, stream=None):
        check(lib().qw3_prefill(self.handle, seq, _ptr(tokens), tokens.numel(), _ptr(logits), _ptr(argmax),
                                _stream(stream)), "qw3_prefill")

    def decode_step(self, tokens, argmax, logits=None, stream=None):
        check(lib().qw3_decode_step(self.handle, _ptr(tokens), _ptr(logits), _ptr(argmax), _stream(stream)),
              "qw3_decode_step")

    def block_forward(self, hidden_in, hidden_out, stream=None):
        check(lib().qw3_block_forward(self.handle, _ptr(hidden_in), hidden_in.shape[0], _ptr(hidden_out),
                                      _stream(stream)), "qw3_block_forward")

    def reset_kv(self, seq=-1):
        check(lib().qw3_reset_kv(self.handle, seq), "qw3_reset_kv")

    def status(self, stream=None):
        return lib().qw3_status_poll(self.handle, _stream(stream))

    def get_len(self, seq=0):
        v = ctypes.c_int32(0)
        check(lib().qw3_get_len(self.handle, seq, ctypes.byref(v)), "qw3_get_len")
        return v.value

    # -------------------------------------------------------------------------------- hooks
    def kv_write(self, seq, layer, pos0, k_bits, v_bits, stream=None):
        check(lib().qw3_kv_write(self.handle, seq, layer, pos0, k_bits.shape[1], _ptr(k_bits), _ptr(v_bits),
                                 _stream(stream)), "qw3_kv_write")

    def kv_read(self, seq, layer, pos0, n_pos, stream=None):
        import torch
        shape = (self.cfg.n_kv_heads, n_pos, self.cfg.head_dim)
        k = torch.empty(shape, dtype=torch.int16, device=self.device)
        v = torch.empty(shape, dtype=torch.int16, device=self.device)
        check(lib().qw3_kv_read(self.handle, seq, layer, pos0, n_pos, _ptr(k), _ptr(v), _stream(stream)),
              "qw3_kv_read")
        return k, v

    def set_len(self, seq, n, stream=None):
        check(lib().qw3_kv_set_len(self.handle, seq, n, _stream(stream)), "qw3_kv_set_len")

    def dequant(self, kind, layer, rows, cols, stream=None):
        import torch
        out = torch.empty((rows, cols), dtype=torch.float32, device=self.device)
        check(lib().qw3_dequant(self.handle, KIND[kind], layer, _ptr(out), _stream(stream)), "qw3_dequant")
        return out

    def bench_kernel(self, kernel, layer=0, reps=1, stream=None):
        check(lib().qw3_bench_kernel(self.handle, kernel, layer, reps, _stream(stream)), "qw3_bench_kernel")

    def close(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.qw3_destroy(self.handle)
        self.handle = None

    def __del__(self):
        self.close()


def canonical_tensors(fmt, embed=None, final_norm=None, layers=(), lm_head=None):
    """ABI tensor list from canonical arrays.

    embed / lm_head: (bf16 bits [V,H]) or (codes [V,H], scales [V,H/32]); final_norm and per-layer norms: bf16
    bits (bf16 format) or f32 (Q8 format); layers: list of dicts slot -> array or (codes, scales)."""
    mdt = DT_Q8 if fmt == WEIGHTS_Q8 else DT_BF16
    ndt = DT_F32 if fmt == WEIGHTS_Q8 else DT_BF16
    out = []

    def mat(kind, layer, m):
        if mdt == DT_Q8:
            out.append(dict(kind=kind, layer=layer, dtype=DT_Q8, data=m[0], scales=m[1]))
        else:
            out.append(dict(kind=kind, layer=layer, dtype=DT_BF16, data=m))

    if embed is not None:
        mat("embed", -1, embed)
        out.append(dict(kind="final_norm", layer=-1, dtype=ndt, data=final_norm))
    if lm_head is not None:
        mat("lm_head", -1, lm_head)
    for l, d in enumerate(layers):
        for slot, v in d.items():
            if slot.endswith("norm"):
                out.append(dict(kind=slot, layer=l, dtype=ndt, data=v))
            else:
                mat(slot, l, v)
    return out
