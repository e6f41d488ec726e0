"""Per-phase timing of the single-launch batch-1 decode (a diagnostic, not part of the library's API).

    python -m transformer_qwen3_block_amd.stamps --build     # on the build host: libqw3_stamps.so, in-tree
    python -m transformer_qwen3_block_amd.stamps [--steps N] # on the GPU: the decode workload, summarised

The stamped build records, for every layer, phase and workgroup, the device clock (s_memrealtime, 100 MHz)
when the phase's inputs had all arrived ("ready") and when the workgroup had published its outputs ("done").
For each phase the summary gives, in microseconds per layer (medians over layers 1..L-1 and the timed steps):
  wait     from the previous phase's last "done" to this phase's first "ready" (exchange latency seen by the
           earliest consumer),
  spread   first to last "ready" across workgroups (how unevenly the inputs arrive),
  work     median per-workgroup "ready" -> "done" (the phase's own compute and publication),
  skew     first to last "done" (what the next phase waits for beyond the median workgroup),
and the layer period (last "done" of D in layer l to the same in layer l+1).
"""
import argparse
import ctypes
import os
import subprocess
import sys

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
STAMPED = os.path.join(_HERE, "libqw3_stamps.so")
PHASES = ("Q", "A", "M", "O", "U", "D")
K_LAYERS, GRID = 64, 256


def build():
    from transformer_qwen3_block_amd import HIPCC_FLAGS, _SOURCES, _ROOT
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    srcs = [os.path.join(_HERE, "csrc", s) for s in _SOURCES]
    cmd = [hipcc, *HIPCC_FLAGS, "-DQW3_MEGA_STAMPS", "-I", os.path.join(_ROOT, "include"), "-I",
           os.path.join(_HERE, "csrc"), *srcs, "-o", STAMPED + ".tmp"]
    subprocess.check_call(cmd)
    os.replace(STAMPED + ".tmp", STAMPED)
    return STAMPED


def summarise(tables, n_layers):
    """tables: list of uint64 arrays [K_LAYERS][6][2][GRID] (one per step)."""
    us = lambda t: t / 100.0  # 100 MHz ticks -> microseconds
    rows = {p: {"wait": [], "spread": [], "work": [], "skew": []} for p in PHASES}
    period = []
    for t in tables:
        t = t.astype(np.int64)
        for l in range(1, n_layers):
            for p in range(6):
                ready, done = t[l, p, 0], t[l, p, 1]
                prev_done = t[l, p - 1, 1] if p > 0 else t[l - 1, 5, 1]
                rows[PHASES[p]]["wait"].append(us(ready.min() - prev_done.max()))
                rows[PHASES[p]]["spread"].append(us(ready.max() - ready.min()))
                rows[PHASES[p]]["work"].append(us(np.median(done - ready)))
                rows[PHASES[p]]["skew"].append(us(done.max() - done.min()))
            period.append(us(t[l, 5, 1].max() - t[l - 1, 5, 1].max()))
    med = {p: {k: float(np.median(v)) for k, v in r.items()} for p, r in rows.items()}
    return med, float(np.median(period))


def run(steps):
    import torch

    import synth
    import transformer_qwen3_block_amd as q
    assert os.path.exists(STAMPED), "build the stamped library first (--build)"
    q._SO = STAMPED
    L = q.lib()
    L.qw3_mega_stamps.restype = ctypes.c_int32
    L.qw3_mega_stamps.argtypes = [ctypes.c_void_p, ctypes.c_uint64]
    wl = synth.Q8_DECODE
    shp = wl.shape
    W = synth.make_weights(shp, seed=wl.seed)
    m = q.Model(q.make_config(**synth.abi_config_kwargs(shp)))
    m.load_weights(synth.abi_tensors(W))
    for l in range(shp.n_layers):
        k, v = synth.kv_fill(wl.seed, 0, l, shp.n_kv_heads, wl.kv_prefill, shp.head_dim)
        m.kv_write(0, l, 0, torch.from_numpy(k.view("int16")).cuda(), torch.from_numpy(v.view("int16")).cuda())
    m.set_len(0, wl.kv_prefill)
    am = torch.tensor(synth.tokens(wl.seed, 1, 1, shp.vocab), dtype=torch.int32, device="cuda")
    side = torch.cuda.Stream()
    buf = np.empty(K_LAYERS * 6 * 2 * GRID, np.uint64)
    tables = []
    with torch.cuda.stream(side):
        for s in range(steps + 4):
            m.decode_step(am, am)
            side.synchronize()
            assert L.qw3_mega_stamps(buf.ctypes.data, buf.nbytes) == 0
            if s >= 4:   # the first steps warm the graph and the caches
                tables.append(buf.reshape(K_LAYERS, 6, 2, GRID).copy())
    assert m.status() == 0
    med, period = summarise(tables, shp.n_layers)
    print(f"single-launch decode, 28-layer Q8, KV context {wl.kv_prefill}: {steps} steps, layers 1..27, "
          f"median layer period {period:.2f} us")
    print(f"{'phase':6}{'wait':>8}{'spread':>8}{'work':>8}{'skew':>8}   (us per layer)")
    for p in PHASES:
        r = med[p]
        print(f"{p:6}{r['wait']:8.2f}{r['spread']:8.2f}{r['work']:8.2f}{r['skew']:8.2f}")
    tot = {k: sum(med[p][k] for p in PHASES) for k in ("wait", "spread", "work", "skew")}
    print(f"{'sum':6}{tot['wait']:8.2f}{tot['spread']:8.2f}{tot['work']:8.2f}{tot['skew']:8.2f}")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--build", action="store_true")
    ap.add_argument("--steps", type=int, default=16)
    a = ap.parse_args()
    if a.build:
        print(build())
    else:
        sys.path.insert(0, os.path.dirname(_HERE))
        run(a.steps)


if __name__ == "__main__":
    main()
