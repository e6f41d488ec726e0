#!/usr/bin/env python3
"""Throughput of the Qwen3-0.6B-shaped decoder on one MI355X, through the C ABI.

Step = one greedy decode token of the 28-layer Qwen3-0.6B shape with Q8 block-32 weights (int8 codes,
one f32 scale per 32 inputs) at batch 1 over a KV context of 2048 positions: embedding, 28 x (RMSNorm +
QKV, QK-Norm + RoPE + KV append + GQA attention, o_proj + residual, RMSNorm + gate/up SwiGLU,
down + residual), final norm, tied logits and argmax.  Inputs are synthetic (seeded PCG32): codes uniform
in [-127,127], scales U(1e-3,1e-2), norms 1+N(0,0.1), KV positions 0..2047 bf16 N(0,1).

Prints one JSON line: decode tok/s (value), end-to-end HBM GB/s, per-kernel times with their achieved
GB/s, the roofline entry of the dominant kernel (HIP events on the launch stream), the bf16 MFMA prefill
of 2048 tokens (prefill tok/s), and the oracle timed on the host cores on a bounded sample.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
F16_MFMA_PEAK_TFLOPS = 2500.0   # MI355X dense f16 / bf16 MFMA (the prefill's operands are f16)


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "decode_q8_b1_ctx2048_hbm_traffic.json")


def counted_traffic(role):
    """HBM bytes per launch of `role` from the committed rocprofv3 counter summary, or None when the kernel
    source changed since the counters were taken."""
    import hashlib
    try:
        prof = json.load(open(TRAFFIC_PROFILE))
    except (OSError, ValueError):
        return None
    for rel, h in prof.get("source_sha256_16", {}).items():
        if hashlib.sha256(open(os.path.join(ROOT, rel), "rb").read()).hexdigest()[:16] != h:
            return None
    k = prof.get("kernels", {}).get(role)
    return k["traffic_bytes"] if k else None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def percentiles(xs):
    import numpy as np
    a = np.asarray(xs, np.float64)
    return {"median": round(float(np.median(a)), 3), "p10": round(float(np.percentile(a, 10)), 3),
            "p90": round(float(np.percentile(a, 90)), 3), "n": int(a.size)}


def timed(torch, stream, fn, reps):
    """Per-call durations (us) of `reps` calls of fn, HIP events on the launch stream around each."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record(stream)
    for i in range(reps):
        fn()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(reps)]


def run_env(torch):
    """What the numbers were measured on: device, ROCm / HIP versions, build flags and the device's clock levels
    (files only: no helper program is started from this GPU process)."""
    import glob
    props = torch.cuda.get_device_properties(0)
    env = {"device": torch.cuda.get_device_name(0), "arch": props.gcnArchName, "cus": props.multi_processor_count,
           "torch": torch.__version__, "hip_runtime": torch.version.hip}
    try:
        env["rocm"] = open("/opt/rocm/.info/version-dev").read().strip()
    except OSError:
        pass
    # current engine / memory clock levels ('*' marks the active one) of the card on this PCI bus
    bus = f"{props.pci_domain_id:04x}:{props.pci_bus_id:02x}:{props.pci_device_id:02x}"
    for dev in glob.glob("/sys/class/drm/card*/device"):
        try:
            if bus not in open(dev + "/uevent").read():
                continue
            env["clocks"] = {k: [ln.strip() for ln in open(f"{dev}/pp_dpm_{k}") if "*" in ln]
                             for k in ("sclk", "mclk")}
        except OSError:
            pass
    import transformer_qwen3_block_amd as q
    env["hipcc_flags"] = " ".join(q.HIPCC_FLAGS)
    return env


def run_probes(torch, q, stream):
    """Attainable peaks on this machine: a plain HBM read stream over 4 GiB (16 times the MALL) and a loop of
    independent f16 MFMA instructions, each timed with HIP events."""
    import ctypes
    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    buf[:: 1 << 20] = 1
    out = torch.empty(65536, dtype=torch.int32, device="cuda:0")
    L = q.lib()
    s = ctypes.c_void_p(stream.cuda_stream)
    # the stream's rate depends on the grid (how the grid-stride addresses fall on the HBM channels): the
    # best of a few grid sizes is the attainable figure
    grids = (384, 512, 768, 2048, 8192)
    per_grid = {}
    for grid in grids:
        def hbm():
            q.check(L.qw3_probe_hbm_read(ctypes.c_void_p(buf.data_ptr()), nbytes, ctypes.c_void_p(out.data_ptr()),
                                         grid, s), "qw3_probe_hbm_read")
        for _ in range(2):
            hbm()
        t = sorted(timed(torch, stream, hbm, 5))
        per_grid[grid] = round(nbytes / t[len(t) // 2] / 1e3, 1)
    del buf
    iters, mgrid, chains = 1024, 4096, 16
    outf = torch.empty(mgrid * 4, dtype=torch.float32, device="cuda:0")

    def mfma():
        q.check(L.qw3_probe_mfma_f16(iters, mgrid, ctypes.c_void_p(outf.data_ptr()), s), "qw3_probe_mfma_f16")
    mfma()
    t_mfma = timed(torch, stream, mfma, 5)
    flops = mgrid * 4 * iters * chains * (2 * 16 * 16 * 32)
    torch.cuda.empty_cache()
    med = lambda t: sorted(t)[len(t) // 2]
    return {"hbm_read_GBps": max(per_grid.values()),
            "hbm_read_GBps_by_grid": {str(g): v for g, v in per_grid.items()},
            "f16_mfma_TFLOPs": round(flops / med(t_mfma) / 1e6, 1),
            "about": "hand-written probes in the same run: 16-byte nontemporal read stream over 4 GiB (grid-stride, "
                     "4 loads in flight per lane; the best of the listed grid sizes), and 16 independent "
                     "v_mfma_f32_16x16x32_f16 chains per wave (4096 workgroups x 4 waves)"}


def decode_kernel_bytes(shp, ctx):
    """Algorithmic HBM bytes of one launch of each decode kernel at batch 1 (weights incl. Q8 scales,
    KV positions read, activation vectors in/out)."""
    H, I, Q, KV, V = shp.hidden, shp.inter, shp.q_dim, shp.kv_dim, shp.vocab
    q8 = shp.fmt in (2, 3)   # Q8 and Q8_0 weights stream the same device layout (int8 codes + f32 scales)

    def w(rows, cols):
        return rows * cols + rows * (cols // 32) * 4 if q8 else rows * cols * 2

    nqkv = Q + 2 * KV
    layer_w = w(nqkv, H) + w(H, Q) + w(2 * I, H) + w(H, I)
    return {
        "decode_layers": shp.n_layers * (layer_w + ctx * shp.n_kv_heads * shp.head_dim * 2 * 2) + 8 * H,
        "qkv_gemv": w(nqkv, H) + 4 * H + 4 * nqkv,
        "attn_decode": ctx * shp.n_kv_heads * shp.head_dim * 2 * 2 + 4 * nqkv + 4 * Q,
        "o_gemv": w(H, Q) + 4 * Q + 8 * H,
        "gateup_gemv": w(2 * I, H) + 4 * H + 4 * I,
        "down_gemv": w(H, I) + 4 * I + 8 * H,
        "lm_head_argmax": w(V, H) + 4 * H + 4 * V,
    }


def run_decode(args, torch, q, synth):
    wl = synth.Q8_DECODE
    shp = wl.shape
    t0 = time.time()
    W = synth.make_weights(shp, seed=wl.seed)
    cfg = q.make_config(**synth.abi_config_kwargs(shp))
    m = q.Model(cfg, device="cuda:0")
    m.load_weights(synth.abi_tensors(W))
    ctx0 = wl.kv_prefill
    for l in range(shp.n_layers):
        k, v = synth.kv_fill(wl.seed, 0, l, shp.n_kv_heads, ctx0, shp.head_dim)
        m.kv_write(0, l, 0, torch.from_numpy(k.view("int16")).cuda(), torch.from_numpy(v.view("int16")).cuda())
    m.set_len(0, ctx0)
    torch.cuda.synchronize()
    log(f"decode workload ready in {time.time() - t0:.1f}s")

    stream = torch.cuda.current_stream()   # a side stream: decode steps replay as captured HIP graphs
    tok = torch.tensor(synth.tokens(wl.seed, 1, 1, shp.vocab), dtype=torch.int32, device="cuda:0")
    am = torch.empty(1, dtype=torch.int32, device="cuda:0")
    m.decode_step(tok, am)
    token_ids = [int(tok.item()), int(am.item())]   # the warm-up's greedy ids, recorded (untimed)
    for _ in range(args.warmup - 1):
        m.decode_step(am, am)
        token_ids.append(int(am.item()))
    torch.cuda.synchronize()
    # one event between consecutive steps: the first-to-last span times exactly `steps` steps, and the spans
    # between neighbours give the per-step distribution
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    wall0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        m.decode_step(am, am)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = ev[0].elapsed_time(ev[-1]) / args.steps
    step_us = percentiles([ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(args.steps)])
    assert m.status() == 0, "numerical failure latched during the timed decode"
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ctx_mid = ctx0 + args.warmup + args.steps // 2
    log(f"decode: {ms * 1e3:.1f} us/token (wall {wall / args.steps * 1e6:.1f} us/token)")

    # per-kernel timing: back-to-back launches of one kernel bracketed by HIP events on the launch stream
    ctx_now = m.get_len(0)
    kb = decode_kernel_bytes(shp, ctx_now + 1)
    if args.kernel_path:
        ids = {"qkv_gemv": 1, "attn_decode": 2, "o_gemv": 3, "gateup_gemv": 4, "down_gemv": 5, "lm_head_argmax": 6}
    else:  # the layer stack is one persistent launch per token
        ids = {"decode_layers": 7, "lm_head_argmax": 6}
    per_step = {k: (1 if k in ("lm_head_argmax", "decode_layers") else shp.n_layers) for k in ids}
    kernels = {}
    reps = args.kernel_reps
    for name, kid in ids.items():
        m.bench_kernel(kid, 0, 3)
        torch.cuda.synchronize()
        e0.record(stream)
        m.bench_kernel(kid, 0, reps)   # enqueued back to back from C++, layers cycling
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        kernels[name] = {"us": round(us, 3), "bytes": kb[name], "GBps": round(kb[name] / us / 1e3, 1),
                         "launches_per_step": per_step[name]}
    step_bytes = sum(decode_kernel_bytes(shp, ctx_mid)[k] * per_step[k] for k in ids)
    dom = max(kernels, key=lambda k: kernels[k]["us"] * kernels[k]["launches_per_step"])
    del m
    torch.cuda.empty_cache()
    return dict(shp=shp, wl=wl, W=W, ms=ms, wall_us=wall / args.steps * 1e6, kernels=kernels, dominant=dom,
                step_bytes=step_bytes, ctx_mid=ctx_mid, step_us=step_us, token_ids=token_ids)


def decode_steps_timed(torch, m, stream, tok, warmup, steps):
    """Greedy decode steps replayed from the argmax buffer; returns the per-step durations (us)."""
    am = torch.empty(1, dtype=torch.int32, device="cuda:0")
    m.decode_step(tok, am)
    for _ in range(warmup - 1):
        m.decode_step(am, am)
    torch.cuda.synchronize()
    t = timed(torch, stream, lambda: m.decode_step(am, am), steps)
    assert m.status() == 0
    return t


def run_bf16_decode(args, torch, q, synth, stream):
    """The 28-layer bf16 workload at batch 1: prefill of its 128-token prompt (HBM-bound at this length), then
    greedy decode from context 128 (contexts 129..)."""
    wl = synth.BF16_DECODE
    shp = wl.shape
    W = synth.make_weights(shp, seed=wl.seed)
    m = q.Model(q.make_config(**synth.abi_config_kwargs(shp)), device="cuda:0")
    m.load_weights(synth.abi_tensors(W))
    del W
    toks = torch.tensor(synth.tokens(wl.seed, 0, wl.prefill, shp.vocab), dtype=torch.int32, device="cuda:0")
    am = torch.empty(1, dtype=torch.int32, device="cuda:0")

    def pre():
        m.reset_kv(0)
        m.prefill(toks, 0, None, am)
    for _ in range(2):
        pre()
    torch.cuda.synchronize()
    tp = timed(torch, stream, pre, 5)
    m.reset_kv(0)
    m.prefill(toks, 0, None, am)
    td = decode_steps_timed(torch, m, stream, am.clone(), 8, min(args.steps, wl.decode - 8))
    H, I, Q, KV, V, L = shp.hidden, shp.inter, shp.q_dim, shp.kv_dim, shp.vocab, shp.n_layers
    wbytes = 2 * (L * (Q * H + 2 * KV * H + H * Q + 3 * I * H) + V * H)
    ctx_mid = wl.prefill + 8 + len(td) // 2
    step_bytes = wbytes + L * KV * 2 * 2 * ctx_mid
    pre_bytes = 2 * L * (Q * H + 2 * KV * H + H * Q + 3 * I * H) + 2 * V * H
    del m
    torch.cuda.empty_cache()
    pd, dd = percentiles(tp), percentiles(td)
    c0 = wl.prefill + 8
    return {"workload": "28-layer Qwen3-0.6B-shape bf16, batch 1: prefill 128 tokens, then greedy decode "
                        f"(timed steps at contexts {c0}..{c0 + len(td) - 1})",
            "decode_tok_s": round(1e6 / dd["median"], 1), "decode_step_us": dd,
            "decode_hbm_GBps": round(step_bytes / dd["median"] / 1e3, 1),
            "decode_frac_hbm_peak": round(step_bytes / dd["median"] / 1e3 / HBM_PEAK_GBS, 4),
            "prefill128_tok_s": round(wl.prefill / pd["median"] * 1e6, 1), "prefill128_us": pd,
            "prefill128_hbm_GBps": round(pre_bytes / pd["median"] / 1e3, 1)}


def run_q8_variant_decode(args, torch, q, synth, stream, fmt, workload):
    """The 28-layer decode at KV context 2048 with the Q8 weights in another weight format."""
    wl = synth.Q8_DECODE
    from dataclasses import replace
    shp = replace(wl.shape, fmt=fmt)
    W = synth.make_weights(shp, seed=wl.seed)
    m = q.Model(q.make_config(**synth.abi_config_kwargs(shp)), device="cuda:0")
    m.load_weights(synth.abi_tensors(W))
    del W
    for l in range(shp.n_layers):
        k, v = synth.kv_fill(wl.seed, 0, l, shp.n_kv_heads, wl.kv_prefill, shp.head_dim)
        m.kv_write(0, l, 0, torch.from_numpy(k.view("int16")).cuda(), torch.from_numpy(v.view("int16")).cuda())
    m.set_len(0, wl.kv_prefill)
    tok = torch.tensor(synth.tokens(wl.seed, 1, 1, shp.vocab), dtype=torch.int32, device="cuda:0")
    td = decode_steps_timed(torch, m, stream, tok, args.warmup, args.steps)
    del m
    torch.cuda.empty_cache()
    d = percentiles(td)
    return {"workload": workload, "tok_s": round(1e6 / d["median"], 1), "step_us": d}


def run_single_block(args, torch, q, synth, stream):
    """The single-block bf16 workload (hidden 1024, one layer, hidden-state input): prefill of 16 positions
    and per-kernel decode times.  Its 31.5 MB of weights stay in the 256 MB MALL between launches, so these
    are cache-resident times, not HBM-bound ones."""
    wl = synth.SINGLE_BLOCK
    shp = wl.shape
    W = synth.make_weights(shp, seed=wl.seed)
    m = q.Model(q.make_config(**synth.abi_config_kwargs(shp)), device="cuda:0")
    m.load_weights(synth.abi_tensors(W))
    hin = torch.from_numpy(synth.hidden_inputs(wl.seed, 0, wl.prefill + 1, shp.hidden)).cuda()
    out = torch.empty((wl.prefill, shp.hidden), dtype=torch.float32, device="cuda:0")

    def pre():
        m.reset_kv(0)
        m.block_forward(hin[:wl.prefill], out)
    for _ in range(2):
        pre()
    torch.cuda.synchronize()
    tp = percentiles(timed(torch, stream, pre, 10))
    res = {"workload": "single Qwen3-0.6B-shape block, bf16, hidden-state input (cache-resident)",
           "prefill16_us": tp}
    names = {1: "qkv_gemv", 2: "attn_decode", 3: "o_gemv", 4: "gateup_gemv", 5: "down_gemv", 7: "block_persistent"}
    kern = {}
    for kid, name in names.items():
        try:
            m.bench_kernel(kid, 0, 3)
        except q.Qw3Error:
            continue
        torch.cuda.synchronize()
        kern[name] = percentiles(timed(torch, stream, lambda: m.bench_kernel(kid, 0, 1), 20))["median"]
    res["decode_kernel_us"] = kern
    del m
    torch.cuda.empty_cache()
    return res


def run_sampler(torch, q, synth, stream):
    """Deterministic sampling over Qwen3's 151,936 logits: top-k 50, top-p 0.9, temperature 0.8, repetition
    penalty 1.1 over a 64-token history, for 1 and 16 rows."""
    res = {}
    for rows in (1, 16):
        lg = torch.from_numpy(synth.logits_rows(9, 0, rows, 151936, 3.0)).cuda()
        hist = torch.from_numpy(synth.tokens(9, 1, rows * 64, 151936).reshape(rows, 64)).cuda()
        smp = q.Sampler(rows, list(range(rows)))
        fn = lambda: smp(lg, 0.8, 50, 0.9, 1.1, hist)
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        res[f"rows{rows}_us"] = percentiles(timed(torch, stream, fn, 20))["median"]
    return res


def run_file_load(torch, q, synth):
    """The weight-file path: the 28-layer model written as a Q8_0 SLM2 file (safetensors container, Q8_0
    matrices and f32 norms, tied lm_head omitted) to a temporary directory, then qw3_inspect_file (header
    validation) and qw3_load_file (validation, read-only mapping, block unpacking and packing, upload) timed.
    The file was just written, so it is read from the page cache: these are not disk figures."""
    import tempfile
    from dataclasses import replace
    from synth import stfile
    wl = synth.Q8_DECODE
    shp = replace(wl.shape, fmt=synth.FMT_Q8_0)
    W = synth.make_weights(shp, seed=wl.seed)
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "qwen3-0.6b-shape.q8_0.slm2")
        stfile.write(path, stfile.model_entries(W, with_lm_head=False), metadata={"format": "pt"})
        del W
        nbytes = os.path.getsize(path)
        t0 = time.perf_counter()
        rep = q.inspect_file(path)
        t_inspect = time.perf_counter() - t0
        m = q.Model(q.make_config(**synth.abi_config_kwargs(shp)), device="cuda:0")
        loads = []
        for _ in range(3):
            t0 = time.perf_counter()
            m.load_file(path)
            torch.cuda.synchronize()
            loads.append(time.perf_counter() - t0)
        del m
        torch.cuda.empty_cache()
    t_load = sorted(loads)[1]
    return {"workload": "28-layer Qwen3-0.6B-shape Q8_0 SLM2 file from the page cache", "file_bytes": nbytes,
            "tensors": rep.n_tensors, "inspect_ms": round(t_inspect * 1e3, 2), "load_ms": round(t_load * 1e3, 1),
            "load_GBps": round(nbytes / t_load / 1e9, 2)}


def run_prefill(args, torch, q, synth):
    wl = synth.BF16_PREFILL
    shp = wl.shape
    W = synth.make_weights(shp, seed=wl.seed)
    m = q.Model(q.make_config(**synth.abi_config_kwargs(shp)), device="cuda:0")
    m.load_weights(synth.abi_tensors(W))
    del W
    toks = torch.tensor(synth.tokens(wl.seed, 0, wl.prefill, shp.vocab), dtype=torch.int32, device="cuda:0")
    am = torch.empty(1, dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream()
    for _ in range(2):
        m.reset_kv(0)
        m.prefill(toks, 0, None, am)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    times = []
    for _ in range(args.prefill_reps):
        m.reset_kv(0)
        e0.record(stream)
        m.prefill(toks, 0, None, am)
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    assert m.status() == 0
    times.sort()
    ms = times[len(times) // 2]
    T = wl.prefill
    H, I, Q, KV, L = shp.hidden, shp.inter, shp.q_dim, shp.kv_dim, shp.n_layers
    linear = 2 * T * L * (H * (Q + 2 * KV) + Q * H + 2 * H * I + I * H)
    attn = 2 * 2 * shp.n_q_heads * shp.head_dim * L * (T * (T + 1) // 2)   # QK^T and PV over j <= i only
    lm = 2 * shp.vocab * H
    flops = linear + attn + lm
    del m
    torch.cuda.empty_cache()
    return dict(tokens=T, ms=ms, tok_s=T / ms * 1e3, flops=flops, tflops=flops / ms / 1e9)


def run_batched(args, torch, q, synth, fmt=None):
    """16 sequences x 8192-position caches, Q8 (or another Q8 weight format): one greedy step per sequence per
    iteration."""
    from dataclasses import replace
    wl = synth.Q8_BATCHED
    shp = wl.shape if fmt is None else replace(wl.shape, fmt=fmt)
    t0 = time.time()
    W = synth.make_weights(shp, seed=wl.seed)
    m = q.Model(q.make_config(**synth.abi_config_kwargs(shp)), device="cuda:0")
    m.load_weights(synth.abi_tensors(W))
    del W
    for s in range(shp.n_seq):
        for l in range(shp.n_layers):
            k, v = synth.kv_fill(wl.seed, s, l, shp.n_kv_heads, wl.kv_prefill, shp.head_dim)
            m.kv_write(s, l, 0, torch.from_numpy(k.view("int16")).cuda(), torch.from_numpy(v.view("int16")).cuda())
        m.set_len(s, wl.kv_prefill)
    torch.cuda.synchronize()
    log(f"batched workload ready in {time.time() - t0:.1f}s")
    stream = torch.cuda.current_stream()
    am = torch.from_numpy(synth.tokens(wl.seed, 1, shp.n_seq, shp.vocab)).cuda()
    warm, iters = 4, args.batched_iters
    for _ in range(warm):
        m.decode_step(am, am)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(iters):
        m.decode_step(am, am)
    e1.record(stream)
    torch.cuda.synchronize()
    assert m.status() == 0
    ms = e0.elapsed_time(e1) / iters
    ctx_mid = wl.kv_prefill + warm + iters // 2
    H, I, Q, KV, V, L = shp.hidden, shp.inter, shp.q_dim, shp.kv_dim, shp.vocab, shp.n_layers
    mats = Q * H + 2 * KV * H + H * Q + 3 * I * H
    wbytes = (L * mats + V * H) * (1 + 4 / 32)
    kvbytes = shp.n_seq * L * shp.n_kv_heads * shp.head_dim * 2 * 2 * (ctx_mid + 1)
    if fmt is not None:  # a variant line: the iteration only
        del m
        torch.cuda.empty_cache()
        return dict(ms=ms, tok_s=shp.n_seq / ms * 1e3, GBps=(wbytes + kvbytes) / ms / 1e6, iters=iters)
    # attention kernel alone (the dominant kernel of this workload)
    m.bench_kernel(2, 0, 3)
    torch.cuda.synchronize()
    e0.record(stream)
    m.bench_kernel(2, 0, 28)
    e1.record(stream)
    torch.cuda.synchronize()
    attn_us = e0.elapsed_time(e1) * 1e3 / 28
    attn_bytes = kvbytes / L
    del m
    torch.cuda.empty_cache()
    return dict(ms=ms, tok_s=shp.n_seq / ms * 1e3, bytes=wbytes + kvbytes, GBps=(wbytes + kvbytes) / ms / 1e6,
                attn_us=attn_us, attn_GBps=attn_bytes / attn_us / 1e3, iters=iters)


def cpu_baseline(res, oracle, budget_s):
    """The oracle as it stands, on the host cores, decoding greedy tokens of the same Q8 workload."""
    import numpy as np
    import synth
    shp, wl, W = res["shp"], res["wl"], res["W"]
    orc = oracle.Model(W, n_seq=1)
    for l in range(shp.n_layers):
        k, v = synth.kv_fill(wl.seed, 0, l, shp.n_kv_heads, wl.kv_prefill, shp.head_dim)
        orc.kv_write(0, l, 0, k, v)
    orc.set_len(0, wl.kv_prefill)
    tok = int(synth.tokens(wl.seed, 1, 1, shp.vocab)[0])
    n = 0
    t0 = time.perf_counter()
    while True:
        rc, tok, _, _ = orc.step(0, tok, want_logits=False)
        assert rc == 0
        n += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    orc.close()
    return {"value": round(n / dt, 4), "unit": "tok/s", "cores": oracle.get_threads(), "kind": "oracle",
            "sample": f"{n} greedy decode tokens of the same 28-layer Q8 workload from KV context "
                      f"{wl.kv_prefill} (strict f32, token by token), {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--kernel-reps", type=int, default=56)
    ap.add_argument("--prefill-reps", type=int, default=5)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-batched", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the attainable-peak probes and the secondary workloads (bf16, Q8_0, single block, "
                         "sampler)")
    ap.add_argument("--batched-iters", type=int, default=16)
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle decode (0 = skip)")
    ap.add_argument("--kernel-path", action="store_true",
                    help="decode kernel by kernel (one launch per step of a layer) instead of one persistent launch")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 256 MiB device copy (reference for HBM counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the sequence-parallel "
              "multi-GPU layout is described, not run.", file=sys.stderr)
        sys.exit(2)
    if args.warmup < 1 or args.steps < 1:
        sys.exit("--warmup and --steps must be >= 1")

    if args.kernel_path:
        os.environ["QW3_NO_MEGA"] = "1"
    import torch

    import synth
    import transformer_qwen3_block_amd as q
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    q.lib()  # fail loudly when the native library is missing

    side = torch.cuda.Stream(device="cuda:0")
    with torch.cuda.stream(side):
        res = run_decode(args, torch, q, synth)
    extra = {}
    if not args.no_extra:
        with torch.cuda.stream(side):
            for key, fn in (("probes", lambda: run_probes(torch, q, side)),
                            ("bf16_b1", lambda: run_bf16_decode(args, torch, q, synth, side)),
                            ("q8_0_b1", lambda: run_q8_variant_decode(
                                args, torch, q, synth, side, synth.FMT_Q8_0,
                                "as the headline, weights given as Q8_0 34-byte blocks (f16 scale); the packer "
                                "widens the scales to f32, so the device streams the same bytes")),
                            ("q8xq8_b1", lambda: run_q8_variant_decode(
                                args, torch, q, synth, side, synth.FMT_Q8_ACT8,
                                "as the headline, with q8 x q8 layer products: activations quantized to int8 "
                                "per 32-block, int8 dot products (lm_head keeps f32 activations)")),
                            ("single_block", lambda: run_single_block(args, torch, q, synth, side)),
                            ("sampler", lambda: run_sampler(torch, q, synth, side)),
                            ("file_load", lambda: run_file_load(torch, q, synth)),
                            ("q8xq8_batched", lambda: dict(
                                workload="16 sequences x KV context 8192 with q8 x q8 layer products (int8 "
                                         "activations, int8 MFMA per 32-block)",
                                **{k: round(v, 4) if isinstance(v, float) else v for k, v in
                                   run_batched(args, torch, q, synth, synth.FMT_Q8_ACT8).items()}))):
                t0 = time.time()
                extra[key] = fn()
                log(f"{key}: {json.dumps(extra[key])} ({time.time() - t0:.1f}s)")
    if args.copy_probe:
        with torch.cuda.stream(side):
            src = torch.ones(64 << 20, dtype=torch.float32, device="cuda:0")
            dst = torch.empty_like(src)
            for _ in range(3):
                dst.copy_(src)
            torch.cuda.synchronize()
            del src, dst
    pre = None
    if not args.no_prefill:
        try:
            with torch.cuda.stream(side):
                pre = run_prefill(args, torch, q, synth)
            log(f"prefill 2048: {pre['ms']:.3f} ms, {pre['tok_s']:.0f} tok/s, {pre['tflops']:.1f} TFLOP/s")
        except q.Qw3Error as e:
            log(f"prefill unavailable: {e}")
    bat = None
    if not args.no_batched:
        with torch.cuda.stream(side):
            bat = run_batched(args, torch, q, synth)
        log(f"batched 16x8192: {bat['ms']:.3f} ms/iteration, {bat['tok_s']:.0f} tok/s, {bat['GBps']:.0f} GB/s; "
            f"attention {bat['attn_us']:.1f} us/layer = {bat['attn_GBps']:.0f} GB/s")
    cpu = None
    if args.cpu_budget > 0:
        import oracle
        cpu = cpu_baseline(res, oracle, args.cpu_budget)
        log(f"oracle: {cpu['value']} tok/s on {cpu['cores']} threads")

    ms = res["ms"]
    tok_s = 1e3 / ms
    dom = res["dominant"]
    dk = res["kernels"][dom]
    out = {
        "metric": "decode tok/s + achieved HBM GB/s (0.6B-shape, B=1, Q8); prefill tok/s",
        "value": round(tok_s, 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "28-layer Qwen3-0.6B-shape decode, batch 1, Q8 block-32 weights (int8 + f32 scale), "
                               "KV context 2048 (bf16)",
                   "hidden": 1024, "layers": 28, "q_heads": 16, "kv_heads": 8, "head_dim": 128, "mlp": 3072,
                   "vocab": 151936, "kv_context_start": res["wl"].kv_prefill},
        "step_us": res["step_us"],
        "token_ids": res["token_ids"],
        "hbm_GBps": round(res["step_bytes"] / ms / 1e6, 1),
        "step_bytes": res["step_bytes"],
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": dk["GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dk["GBps"] / HBM_PEAK_GBS, 4), "traffic": counted_traffic(dom)},
        "kernels": res["kernels"],
        "cpu_baseline": cpu,
    }
    if pre is not None:
        out["prefill"] = {"workload": "28-layer Qwen3-0.6B-shape bf16-weight prefill of 2048 tokens, batch 1, on "
                                      "f16-operand MFMA (f32 accumulation)",
                          "tok_s": round(pre["tok_s"], 1), "ms": round(pre["ms"], 4),
                          "TFLOPs": round(pre["tflops"], 2), "flop": pre["flops"],
                          "frac_f16_mfma_peak": round(pre["tflops"] / F16_MFMA_PEAK_TFLOPS, 4)}
    if bat is not None:
        out["batched"] = {"workload": "28-layer Qwen3-0.6B-shape Q8 decode, 16 sequences x KV context 8192",
                          "tok_s": round(bat["tok_s"], 1), "ms_per_iteration": round(bat["ms"], 4),
                          "hbm_GBps": round(bat["GBps"], 1), "attn_us_per_layer": round(bat["attn_us"], 2),
                          "attn_GBps": round(bat["attn_GBps"], 1), "iterations": bat["iters"]}
    probes = extra.pop("probes", None)
    if probes:
        out["roofline"]["attainable_peak"] = probes["hbm_read_GBps"]
        out["roofline"]["frac_attainable"] = round(dk["GBps"] / probes["hbm_read_GBps"], 4)
        out["probes"] = probes
        if pre is not None:
            out["prefill"]["frac_attainable_mfma"] = round(pre["tflops"] / probes["f16_mfma_TFLOPs"], 4)
    out.update(extra)
    out["env"] = run_env(torch)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
