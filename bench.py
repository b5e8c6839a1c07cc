#!/usr/bin/env python3
"""Benchmark: CommVQ decode-step attention, KV tokens/s per layer at 128K context (1-bit and 2-bit).

One step = one decode-step attention call for one layer (every row of the hot path: code stream and
unpack, RoPE phases, key scores, split softmax, value reduce, combine) on the Llama-3.1-8B layer shape
(8 KV / 32 q heads, head dim 128, G = 16, N = 256). Steps rotate over `layers` distinct copies of the
layer's codes, codebooks and query (>= 1 GiB in total) so the 256 MB Infinity Cache cannot serve
the code stream. Inputs are synthetic (workloads.make_inputs) and resident in HBM before timing.

Before anything is timed, every layer copy is launched once and the workload runs for 1 s (untimed), so that
buffers have been touched and the GPU clocks have settled; then the W warmup steps. The timed region is K
back-to-back steps between two device synchronizations, bracketed by HIP events on the launch stream: its
average is the kernel's duration for the roofline (rocprofv3's kernel trace of the same command agrees).
Each launch is also timed alone between its own two events (us_per_launch_isolated, an upper bound: the
events add a few microseconds). Measurement probes (libcommvq_probes.so) give the HBM read rate a plain
streaming kernel reaches and the LDS random-gather ceiling. cpu_baseline times the fp64 oracle on the host
on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads  # noqa: E402

HBM_PEAK_GBPS = 8000.0
# LDS: 256 CUs x 256 B per clock x 2.4 GHz (a broadcast ds_read_b128 wave instruction, 1 KiB, takes 4 clocks
# per CU). The random 16-byte gathers the kernels make run slower (bank conflicts): their ceiling is measured
# live by commvq_probe_lds_gather (lds_gather_probe below).
LDS_PEAK_TBPS = 256 * 256 * 2.4e9 / 1e12
CLOCK_GHZ = 2.4
# MI355X fp32 vector peak as published (it counts packed fp32 instructions, which this build does not use:
# without them the VALU fp32 rate is half, 78.6 TFLOP/s)
FP32_VECTOR_PEAK_TFLOPS = 157.3
PROFILES = os.path.join(ROOT, "profiles")
# the attention kernel of each workload family, as rocprofv3 names it, and the sources that determine it
_CSRC = os.path.join(ROOT, "vector_quantized_kv_amd", "csrc")
_COMMON = ("attn_common.h", "commvq_internal.h", "device_common.h", "api.cpp")
KERNELS = {
    "f16": ("attn_f16_kernel", [os.path.join(_CSRC, f) for f in ("attn_f16.hip",) + _COMMON]),
    "f32": ("attn_f32_kernel", [os.path.join(_CSRC, f) for f in ("attn.hip",) + _COMMON]),
    "wide": ("attn_wide_kernel", [os.path.join(_CSRC, f) for f in ("attn_wide.hip",) + _COMMON]),
}


def kernel_kind(cfg) -> str:
    return "wide" if cfg.packed else ("f16" if cfg.dtype == "float16" else "f32")


def kernel_label(cfg) -> str:
    """The kernel's name as rocprofv3 reports it: byte layout templated on R, bit-packed layout on the number of
    residuals in the last 8-residual index window."""
    name = KERNELS[kernel_kind(cfg)][0]
    R = cfg.n_residuals
    return f"{name}<{R - 8 * ((R + 7) // 8 - 1)}>" if cfg.packed else f"{name}<{R}>"


def kernel_source_hash(kind: str) -> str:
    h = hashlib.sha256()
    for p in KERNELS[kind][1]:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(cfg):
    """HBM bytes per launch from the committed rocprofv3 PMC summary, if it matches the current kernel."""
    path = os.path.join(PROFILES, f"traffic_attn_decode_{cfg.name}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != kernel_source_hash(kernel_kind(cfg)):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def algorithmic_bytes(cfg, total_tokens: int) -> dict:
    """Bytes the method must move per call. Code stream: K and V, R bytes per group, G groups."""
    codes = workloads.code_bytes(cfg, total_tokens)
    esize = 2 if cfg.dtype == "float16" else 4
    codebooks = 2 * cfg.n_kv_heads * cfg.n_groups * cfg.n_residuals * cfg.n_codes * cfg.group_dim * esize
    q = cfg.batch * cfg.n_q_heads * cfg.head_dim * esize
    out = cfg.batch * cfg.n_q_heads * cfg.head_dim * 4
    return {"codes": codes, "codebooks": codebooks, "q_out": q + out, "total": codes + codebooks + q + out}


def host_info() -> dict:
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "host_logical_cpus": os.cpu_count(), "cpus_available": len(os.sched_getaffinity(0))}


def cpu_baseline(cfg, inp, budget_s: float = 12.0) -> dict:
    import oracle
    cores = len(os.sched_getaffinity(0))
    threads = min(cores, 16)
    d_tokens = int(inp["total_tokens"])
    runs, t_total = 0, 0.0
    while True:
        t0 = time.perf_counter()
        oracle.run_config(cfg, inp, n_threads=threads)
        t_total += time.perf_counter() - t0
        runs += 1
        if t_total * threads >= budget_s or runs >= 20:
            break
    per_run = t_total / runs
    res = {"value": d_tokens / per_run, "unit": "KV tokens/s per layer", "cores": threads, "kind": "oracle",
           "sample": f"{runs} full decode steps of one layer ({cfg.name}: {d_tokens} tokens x "
                     f"{cfg.n_kv_heads} KV heads), fp64, {threads} host threads; {per_run:.3f} s per step"}
    res.update(host_info())
    # the same oracle on one thread, on the small workloads the tests use
    single = {}
    for name in ("tiny_1k_r2_f32", "llama8b_8k_r2"):
        c = workloads.CONFIGS[name]
        x = workloads.make_inputs(c)
        t0 = time.perf_counter()
        oracle.run_config(c, x, n_threads=1)
        dt = time.perf_counter() - t0
        single[name] = {"s_per_step": dt, "kv_tokens_per_s": int(x["total_tokens"]) / dt}
    res["single_thread"] = single
    return res


def probes_lib():
    import ctypes
    from vector_quantized_kv_amd import build as vbuild
    L = ctypes.CDLL(vbuild.PROBES_LIB)
    L.commvq_probe_read_stream.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p,
                                           ctypes.c_void_p]
    L.commvq_probe_lds_gather.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    L.commvq_probe_lds_bin_add.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    return L


def settle(launch, seconds: float = 1.0):
    """Keeps the GPU busy with `launch` for `seconds` of wall time (untimed): the device raises its clocks
    over the first tens of milliseconds of load, and a kernel timed before that runs up to 15% slower."""
    import torch
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < seconds:
        launch(i)
        i += 1
        if i % 64 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def _timed_ms(fn, reps: int) -> float:
    import torch
    fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def read_stream_probe(nbytes: int = 1 << 30, reps: int = 10) -> dict:
    """HBM read rate a plain streaming kernel reaches on this device (commvq_probe_read_stream: 16-byte
    non-temporal loads, 2048 workgroups of 256 threads, over a 1 GiB buffer)."""
    import torch
    L = probes_lib()
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream

    def run():
        assert L.commvq_probe_read_stream(buf.data_ptr(), nbytes, 2048, sink.data_ptr(), s) == 0
    settle(lambda i: run(), 0.5)
    ms = _timed_ms(run, reps)
    del buf
    return {"GBps": nbytes / (ms * 1e-3) * 1e-9, "bytes": nbytes, "kernel": "read_stream_kernel"}


def lds_gather_probe(iters: int = 256, blocks: int = 1024, reps: int = 5) -> dict:
    """Random 16-byte LDS row gathers (commvq_probe_lds_gather: one workgroup of 8 waves per CU, each wave
    gathering from a 64 KiB table of 16 groups x 256 rows, a random row per lane): the ceiling of the
    attention kernels' codebook reads."""
    import torch
    L = probes_lib()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream

    def run():
        assert L.commvq_probe_lds_gather(iters, blocks, sink.data_ptr(), s) == 0
    settle(lambda i: run(), 0.5)
    ms = _timed_ms(run, reps)
    gathers = blocks * 8 * iters * 16  # wave instructions, 1 KiB each
    tbps = gathers * 1024 / (ms * 1e-3) * 1e-12
    return {"TBps": tbps, "clk_per_wave_gather_per_cu_at_2.4GHz": 256 * 1024 * CLOCK_GHZ * 1e9 / (tbps * 1e12),
            "kernel": "lds_gather_kernel", "gathers": gathers}


def lds_bin_add_probe(iters: int = 64, blocks: int = 1024, reps: int = 5) -> dict:
    """Random 64-bit LDS atomic adds (commvq_probe_lds_bin_add: one workgroup of 8 waves per CU, bins of 42 units
    x 2 head pairs x 64 codewords, a random codeword per lane): the ceiling of the bit-packed kernel's value
    bins. The bins' total is checked against the number of adds."""
    import torch
    L = probes_lib()
    sink = torch.zeros(1, dtype=torch.int64, device="cuda")
    s = torch.cuda.current_stream().cuda_stream

    def run():
        assert L.commvq_probe_lds_bin_add(iters, blocks, sink.data_ptr(), s) == 0
    sink.zero_()
    run()
    torch.cuda.synchronize()
    adds = blocks * 8 * iters * 42 * 2  # wave instructions, 64 lanes each
    assert int(sink.item()) == adds * 64, "LDS bin-add probe: the bins do not hold every add"
    settle(lambda i: run(), 0.5)
    ms = _timed_ms(run, reps)
    return {"G_wave_adds_per_s": adds / (ms * 1e-3) * 1e-9,
            "clk_per_wave_add_per_cu_at_2.4GHz": 256 * CLOCK_GHZ * 1e9 * (ms * 1e-3) / adds,
            "kernel": "lds_bin_add_kernel", "wave_adds": adds}


def profile_run(names, launches: int):
    """Few launches per workload (for rocprofv3), after one setup launch per layer copy, plus a 1 GiB device copy
    whose FETCH_SIZE / WRITE_SIZE calibrate the counters (it reads and writes exactly 1 GiB), plus the probes."""
    import torch
    import vector_quantized_kv_amd as vq
    for name in names:
        cfg = workload(name)
        d = vq.dims_of(cfg)
        base = workloads.make_inputs(cfg)
        per_layer = algorithmic_bytes(cfg, int(base["total_tokens"]))["total"]
        layers = max(4, int(math.ceil((1 << 30) / per_layer)))
        rope = vq.rope_table(d, int(base["max_len"]))
        same_lengths = dataclasses.replace(cfg, lengths=tuple(int(x) for x in base["seq_len"]), ragged_range=None)
        Ls = [vq.Layer(d, base if i == 0 else workloads.make_inputs(same_lengths, seed=cfg.seed + 1000 * i),
                       rope=rope, rope_positions=int(base["max_len"])) for i in range(layers)]
        share_descriptors(Ls)
        for ly in Ls:  # every layer copy once (setup; also the first touch of its buffers)
            ly.attn_decode()
        torch.cuda.synchronize()
        settle(lambda i: Ls[i % layers].attn_decode())
        # as bench.py times launches: each between two HIP events on the launch stream
        stream = torch.cuda.current_stream()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(launches)]
        for i in range(launches):
            ev[i][0].record(stream)
            Ls[i % layers].attn_decode()
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        print(f"profile: {name} {layers} setup launches, 1 s of launches, then {launches} launches over {layers} "
              "layer copies", flush=True)
        del Ls
        torch.cuda.empty_cache()
    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print("profile: 3 copies of 1 GiB (calibration)", flush=True)
    del src, dst
    torch.cuda.empty_cache()
    read_stream_probe(reps=3)
    lds_gather_probe(reps=3)
    lds_bin_add_probe(reps=3)
    print("profile: probes (read stream, LDS gathers, LDS bin adds: 0.5 s of launches, then 1 + 3 more each)",
          flush=True)


def share_descriptors(Ls):
    """The layer copies of one decode step serve the same batch: like the RoPE table, the sequence descriptors
    (seq_start, seq_len; equal in every copy) are one pair of device arrays shared by all of them, as in a
    model, where every layer reads the same ones."""
    for ly in Ls[1:]:
        assert bool((ly.seq_start == Ls[0].seq_start).all()) and bool((ly.seq_len == Ls[0].seq_len).all())
        ly.seq_start, ly.seq_len = Ls[0].seq_start, Ls[0].seq_len


def run_config(cfg, steps: int, warmup: int, layers: int, use_graph: bool, check: bool, probes: dict):
    import torch
    import vector_quantized_kv_amd as vq

    d = vq.dims_of(cfg)
    base = workloads.make_inputs(cfg)
    total = int(base["total_tokens"])
    per_layer = algorithmic_bytes(cfg, total)
    if layers <= 0:
        layers = max(4, int(math.ceil((1 << 30) / per_layer["total"])))
    rope = vq.rope_table(d, int(base["max_len"]))
    # the rotated copies keep the first copy's sequence lengths (a ragged workload would otherwise draw new
    # ones per copy) and draw new codes, codebooks and queries
    same_lengths = dataclasses.replace(cfg, lengths=tuple(int(x) for x in base["seq_len"]), ragged_range=None)
    Ls = []
    for i in range(layers):
        inp = base if i == 0 else workloads.make_inputs(same_lengths, seed=cfg.seed + 1000 * i)
        Ls.append(vq.Layer(d, inp, rope=rope, rope_positions=int(base["max_len"])))
    share_descriptors(Ls)
    torch.cuda.synchronize()
    check_err = None
    if check:
        import oracle
        got = Ls[0].attn_decode().cpu().numpy().astype(np.float64)
        ref = oracle.run_config(cfg, base, n_threads=min(len(os.sched_getaffinity(0)), 16))
        check_err = float((np.abs(got - ref).max(-1) / np.abs(ref).max(-1)).max())

    stream = torch.cuda.current_stream()
    # setup (untimed): every rotated layer copy is launched once (first touch of its buffers), then the workload
    # runs for 1 s so that the GPU clocks have settled, then the W warmup steps
    for ly in Ls:
        ly.attn_decode()
    torch.cuda.synchronize()
    settle(lambda i: Ls[i % layers].attn_decode())
    for i in range(warmup):
        Ls[i % layers].attn_decode()
    torch.cuda.synchronize()

    # timed region: K back-to-back steps between two device synchronizations
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(steps):
        Ls[i % layers].attn_decode()
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)

    # each launch alone between its own two events: an upper bound on the kernel's duration (the events add
    # their own per-launch work, a few microseconds); reported beside the timed region's average
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        ev[i][0].record(stream)
        Ls[i % layers].attn_decode()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    launch_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))

    graph_ms = None
    if use_graph:
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            Ls[0].attn_decode()  # warm the capture stream
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for i in range(layers):
                Ls[i].attn_decode()
        # the replays run for 0.5 s before the timed ones, and at least 20 replays are timed: a single replay
        # also times the graph launch and reads up to 15% slow at 128K
        settle(lambda i: g.replay(), 0.5)
        reps = max(20, steps // layers)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        graph_ms = a.elapsed_time(b) / (reps * layers)

    # the kernel's average duration (one launch per step): the timed region over K, HIP events on the launch
    # stream (rocprofv3's kernel trace of the same command agrees with it)
    per_step_ms = total_ms / steps
    print(f"[bench] {cfg.name}: {layers} layers, {per_step_ms * 1e3:.1f} us per step ({launch_ms * 1e3:.1f} us per "
          "launch timed alone)", file=sys.stderr, flush=True)
    L = total
    res = {
        "config": cfg.name, "tokens": L, "layers_rotated": layers, "ms_per_step": per_step_ms,
        "us_per_layer_eager": per_step_ms * 1e3, "us_per_launch_isolated": launch_ms * 1e3,
        "us_per_layer_graph": None if graph_ms is None else graph_ms * 1e3,
        "kv_tokens_per_s_per_layer": L / (per_step_ms * 1e-3),
        "code_stream_GBps": per_layer["codes"] / (per_step_ms * 1e-3) * 1e-9,
        "compulsory_GBps": per_layer["total"] / (per_step_ms * 1e-3) * 1e-9,
        "pct_hbm_peak_code_stream": 100.0 * per_layer["codes"] / (per_step_ms * 1e-3) * 1e-9 / HBM_PEAK_GBPS,
        "bytes": per_layer, "max_row_rel_err_vs_oracle": check_err,
    }
    # Byte layout: every token gathers, per residual and group, its 16-byte codeword row from LDS for keys and
    # again for values; that LDS stream is what bounds the kernel. Bit-packed layout: the keys gather 128-byte
    # rows the same way, and the values make two random 64-bit LDS adds per (token, residual, group) into the
    # bins; its LDS floor is the key gathers at the measured gather ceiling plus the adds at the measured add
    # ceiling. The whole launch, fixed costs included, is counted against them.
    gather_tbps = probes["lds_random_gather"]["TBps"]
    row_bytes = cfg.group_dim * (2 if cfg.dtype == "float16" else 4)
    units = cfg.n_kv_heads * L * cfg.n_residuals * cfg.n_groups  # (token, KV head, residual, group)
    if cfg.packed:
        key_bytes = units * row_bytes
        wave_adds = 2 * units / 64
        clk_add = probes["lds_bin_add"]["clk_per_wave_add_per_cu_at_2.4GHz"]
        floor_s = key_bytes / (gather_tbps * 1e12) + wave_adds * clk_add / (256 * CLOCK_GHZ * 1e9)
        res["lds_roofline"] = {"bound": "lds", "key_gathered_bytes_per_launch": key_bytes,
                               "value_bin_adds_per_launch": 2 * units, "random_gather_ceiling_TBps": gather_tbps,
                               "bin_add_clk_per_wave_instruction": clk_add, "floor_us": floor_s * 1e6,
                               "frac_of_lds_floor": floor_s / (per_step_ms * 1e-3)}
    else:
        gathered = 2 * units * row_bytes
        tbps = gathered / (per_step_ms * 1e-3) * 1e-12
        res["lds_roofline"] = {"bound": "lds", "gathered_bytes_per_launch": gathered, "achieved": tbps,
                               "unit": "TB/s", "peak": LDS_PEAK_TBPS, "frac": tbps / LDS_PEAK_TBPS,
                               "random_gather_ceiling": gather_tbps,
                               "frac_of_random_gather_ceiling": tbps / gather_tbps}
    res["kernel"] = kernel_label(cfg)
    res["hbm_traffic_bytes_per_launch"] = read_traffic(cfg)
    del Ls
    torch.cuda.empty_cache()
    return res, base


def codebook_tools_timing(reps: int = 3):
    """The offline steps next to the decode path, at the 128K layer shape (8 KV heads, R = 2, fp16):
    encoding every cached key of a 131072-token prefill with commvq_encode_greedy, one codebook M-step
    (commvq_codebook_update) over the same tokens, and the same prefill encoded into bit-packed records (R = 21)
    with one M-step over them. Per (token, KV head, group, round) the encoder evaluates
    256 squared distances of 8 dims (8 subtractions + 8 multiply-adds = 24 flops each, fp32 VALU)."""
    import torch
    import vector_quantized_kv_amd as vq
    Hkv, n, R = 8, 131072, 2
    g = torch.Generator(device="cuda").manual_seed(123)
    x = (torch.randn((Hkv, n, 128), generator=g, device="cuda") * 0.7).half()
    cb = (torch.randn((Hkv, 16, R, 256, 8), generator=g, device="cuda") * 0.5).half()
    d = vq.make_dims(1, 4 * Hkv, Hkv, R, "float16")
    codes = vq.encode_greedy(d, x, cb)
    out = vq.codebook_update(d, x, codes, cb)
    torch.cuda.synchronize()
    def timed(fn):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps * 1e-3
    t_enc = timed(lambda: vq.encode_greedy(d, x, cb, codes=codes))
    t_upd = timed(lambda: vq.codebook_update(d, x, codes, cb, codebook_out=out))
    enc_flops = float(Hkv) * n * 16 * R * 256 * 24
    # the same prefill encoded into bit-packed records (one index per 64 dims, N = 64, R = 21): per (token,
    # KV head, group, round) 64 squared distances of 64 dims (3 flops per dim)
    Rb = 21
    cbb = (torch.randn((Hkv, 2, Rb, 64, 64), generator=g, device="cuda") * 0.5).half()
    db = vq.make_dims(1, 4 * Hkv, Hkv, Rb, "float16", n_groups=2, n_codes=64)
    words = vq.encode_greedy(db, x, cbb)
    outb = vq.codebook_update(db, x, words, cbb)
    torch.cuda.synchronize()
    t_encb = timed(lambda: vq.encode_greedy(db, x, cbb, codes=words))
    t_updb = timed(lambda: vq.codebook_update(db, x, words, cbb, codebook_out=outb))
    encb_flops = float(Hkv) * n * 2 * Rb * 64 * 64 * 3
    return {
        "shape": f"{n} tokens x {Hkv} KV heads, R={R}, fp16",
        # against the published fp32 vector peak (157.3 TFLOP/s, which assumes packed fp32 instructions; this
        # build does not use them, so 0.5 is the most it can reach)
        "encode_greedy": {"ms": t_enc * 1e3, "tokens_per_s": n / t_enc, "bound": "alu",
                          "achieved_tflops": enc_flops / t_enc * 1e-12, "peak_tflops": FP32_VECTOR_PEAK_TFLOPS,
                          "frac": enc_flops / t_enc * 1e-12 / FP32_VECTOR_PEAK_TFLOPS},
        "codebook_update": {"ms": t_upd * 1e3, "tokens_per_s": n / t_upd},
        "encode_greedy_bit_packed_r21": {"ms": t_encb * 1e3, "tokens_per_s": n / t_encb, "bound": "alu",
                                         "achieved_tflops": encb_flops / t_encb * 1e-12,
                                         "peak_tflops": FP32_VECTOR_PEAK_TFLOPS,
                                         "frac": encb_flops / t_encb * 1e-12 / FP32_VECTOR_PEAK_TFLOPS},
        "codebook_update_bit_packed_r21": {"ms": t_updb * 1e3, "tokens_per_s": n / t_updb},
    }


def step_kernels_timing(probes: dict, reps: int = 20):
    """The exported steps of the path, each on its own at the 128K layer shape (llama8b_128k_r2 inputs, fp16,
    R = 2), against the HBM roofline of its algorithmic bytes: the RoPE phase table for 131072 positions (bytes
    written), the query x codebook table of the 32 q heads (codebook read, table written), and the value reduction
    (value codes and fp32 weights p read; bins in LDS, one partial per 2048-token split, then their sum). The value
    reduction's binning makes one random 64-bit LDS add per (token, KV head, group, residual, head pair) (the
    weights here are non-negative, so two heads share a bin word); at the live bin-add probe's rate those adds
    alone take `lds_floor_us`, the bound that this step actually meets. `pages_setting` times the same two table
    steps on the pages' own bit-packed layout (64-dim groups, 64 codewords, R = 21) at the same context.
    `reps` launches of each are captured in one HIP graph and the replay is timed, so the figure is the kernels'
    own time and not the host's launch rate (the table kernels run for a few microseconds)."""
    import torch
    import vector_quantized_kv_amd as vq
    cfg = workloads.CONFIGS["llama8b_128k_r2"]
    d = vq.dims_of(cfg)
    inp = workloads.make_inputs(cfg)
    ly = vq.Layer(d, inp)
    T = int(inp["total_tokens"])
    g = torch.Generator(device="cuda").manual_seed(7)
    p = torch.rand((cfg.batch, cfg.n_q_heads, ly.max_len), generator=g, device="cuda")
    rope = vq.rope_table(d, T)
    table = vq.qcodebook_table(d, ly.q, ly.k_cb)
    vout = vq.value_reduce(d, p, ly.v_codes, ly.v_cb, ly.seq_start, ly.seq_len, ly.max_len, T)
    ws = torch.empty(max(vq.value_reduce_workspace_size(d, ly.max_len), 16), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()

    def timed(fn):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(reps):
                fn()
        settle(lambda i: graph.replay(), 0.2)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(5):
            graph.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / (5 * reps) * 1e-3

    def line(t, nbytes):
        gbps = nbytes / t * 1e-9
        return {"us": t * 1e6, "algorithmic_bytes": nbytes, "achieved_GBps": gbps, "bound": "hbm",
                "peak_GBps": HBM_PEAK_GBPS, "frac": gbps / HBM_PEAK_GBPS}
    t_rope = timed(lambda: vq.rope_table(d, T, out=rope))
    t_tab = timed(lambda: vq.qcodebook_table(d, ly.q, ly.k_cb, out=table))
    t_val = timed(lambda: vq.value_reduce(d, p, ly.v_codes, ly.v_cb, ly.seq_start, ly.seq_len, ly.max_len, T,
                                          workspace=ws, out=vout))
    cb_bytes = ly.k_cb.numel() * ly.k_cb.element_size()
    # the pages' own setting: bit-packed records, R = 21, the same context and heads
    pcfg = workloads.PAGES_CONFIGS["pages_g64_r21_128k"]
    pd = vq.dims_of(pcfg)
    pinp = workloads.make_inputs(pcfg)
    ply = vq.Layer(pd, pinp)
    ptable = vq.qcodebook_table(pd, ply.q, ply.k_cb)
    pvout = vq.value_reduce(pd, p, ply.v_codes, ply.v_cb, ply.seq_start, ply.seq_len, ply.max_len, T)
    pws = torch.empty(max(vq.value_reduce_workspace_size(pd, ply.max_len), 16), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    t_ptab = timed(lambda: vq.qcodebook_table(pd, ply.q, ply.k_cb, out=ptable))
    t_pval = timed(lambda: vq.value_reduce(pd, p, ply.v_codes, ply.v_cb, ply.seq_start, ply.seq_len, ply.max_len, T,
                                           workspace=pws, out=pvout))
    pcb_bytes = ply.k_cb.numel() * ply.k_cb.element_size()
    pages = {
        "shape": f"{T} tokens, {pcfg.n_kv_heads} KV / {pcfg.n_q_heads} q heads, bit-packed, G=2, N=64, "
                 f"R={pcfg.n_residuals}, fp16",
        "qcodebook_table": line(t_ptab, pcb_bytes + ptable.numel() * ptable.element_size()),
        "value_reduce": dict(line(t_pval, ply.v_codes.numel() * ply.v_codes.element_size() + p.numel() * 4),
                             **lds_adds_floor(2 * T * pcfg.n_kv_heads * pcfg.n_groups * pcfg.n_residuals, t_pval,
                                              probes)),
    }
    return {
        "shape": f"{T} tokens, {cfg.n_kv_heads} KV / {cfg.n_q_heads} q heads, R={cfg.n_residuals}, fp16",
        "timing": f"{reps} launches in one HIP graph, 5 replays",
        "rope_table": line(t_rope, rope.numel() * 4),
        "qcodebook_table": line(t_tab, cb_bytes + table.numel() * table.element_size()),
        "value_reduce": dict(line(t_val, ly.v_codes.numel() * ly.v_codes.element_size() + p.numel() * 4),
                             **lds_adds_floor(2 * T * cfg.n_kv_heads * cfg.n_groups * cfg.n_residuals, t_val, probes)),
        "pages_setting": pages,
    }


def lds_adds_floor(lane_adds: int, seconds: float, probes: dict) -> dict:
    """LDS floor of `lane_adds` random 64-bit LDS adds (64 per wave instruction) at the bin-add probe's measured
    cost per wave instruction per CU, over 256 CUs at 2.4 GHz."""
    clk = probes["lds_bin_add"]["clk_per_wave_add_per_cu_at_2.4GHz"]
    floor_s = lane_adds / 64 * clk / (256 * CLOCK_GHZ * 1e9)
    return {"lds_bin_adds": lane_adds, "bin_add_clk_per_wave_instruction": clk, "lds_floor_us": floor_s * 1e6,
            "frac_of_lds_floor": floor_s / seconds}


# workloads of bench.py --profile (one attention kernel per workload kind; 20 launches each)
PROFILE_ALSO = ("llama8b_128k_r1", "pages_g64_r11_128k", "pages_g64_r21_128k")

# The pages' only absolute timing of this path, next to the workload it is closest to: per-layer decode
# latency at 8K context, naive (decode the codes, then attend) and with the commutative codebook
# ("CommVQ: Commutative Vector Quantization for KV Cache Compression" summary page, measured-effects table;
# the paper's Table 5 as the pith.science referee report describes it). No GPU, model or batch is named.
PAGES_CONTEXT = {
    "llama8b_8k_r2": {"per_layer_latency_us": {"naive": 2400.0, "commutative_codebook": 400.0},
                      "hardware": "not named on the pages", "role": "context, not a target"},
}


def _csv_rows(directory: str, suffix: str):
    """Rows of the rocprofv3 csv file *<suffix> (or *<suffix>.gz) under directory."""
    import csv
    import glob
    import gzip
    import io
    paths = sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True) +
                   glob.glob(os.path.join(directory, "**", f"*{suffix}.gz"), recursive=True))
    if not paths:
        raise SystemExit(f"no *{suffix} under {directory}")
    if paths[0].endswith(".gz"):
        with gzip.open(paths[0], "rt", newline="") as f:
            return list(csv.DictReader(io.StringIO(f.read())))
    with open(paths[0], newline="") as f:
        return list(csv.DictReader(f))


def _dispatches(rows, value_key=None):
    """[(kernel name, value or duration ns)] in dispatch order, one entry per dispatch."""
    out = {}
    for r in rows:
        did = int(r.get("Dispatch_Id") or r.get("Dispatch_ID") or r.get("Correlation_Id"))
        name = r["Kernel_Name"]
        if value_key is None:
            v = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        else:
            v = float(r[value_key])
            if did in out:
                v += out[did][1]  # a counter summed over its instances
        out[did] = (name, v)
    return [out[k] for k in sorted(out)]


PROFILE_LAUNCHES = 20  # launches per workload in the bench.py --profile runs the summaries are made from


def _profiled_dispatches(seq, cfgs, launches: int) -> dict:
    """Per workload of a bench.py --profile run, its profiled attention dispatches: each workload starts with its
    RoPE table (one rope_table_kernel dispatch), and its profiled launches are the last `launches` attention
    dispatches before the next workload."""
    segs, cur = [], None
    for x in seq:
        if "rope_table_kernel" in x[0]:
            cur = []
            segs.append(cur)
        elif cur is not None and "attn_" in x[0] and "_kernel" in x[0]:
            cur.append(x)
    assert len(segs) == len(cfgs), (len(segs), len(cfgs))
    return {c.name: seg[-launches:] for c, seg in zip(cfgs, segs)}


SQ_PASSES = (
    "SQ_WAVE_CYCLES SQ_BUSY_CU_CYCLES SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS SQ_ACTIVE_INST_ANY SQ_WAIT_INST_LDS "
    "SQ_WAIT_INST_ANY SQ_VALU_MFMA_BUSY_CYCLES",
    "SQ_INSTS_VALU SQ_INSTS_LDS SQ_INSTS_MFMA SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_INST_LEVEL_LDS "
    "SQ_LDS_DATA_FIFO_FULL SQ_LDS_CMD_FIFO_FULL",
)


def write_counters(dirs):
    """profiles/sq_counters_attn_128k.md from two rocprofv3 --pmc runs of bench.py --profile (SQ_PASSES)."""
    import collections
    names = ["llama8b_128k_r2"] + [n for n in PROFILE_ALSO if n != "llama8b_128k_r2"]
    cfgs = [workload(n) for n in names]
    vals = collections.defaultdict(dict)
    for d in dirs:
        rows = _csv_rows(d, "counter_collection.csv")
        for counter in sorted({r["Counter_Name"] for r in rows}):
            seq = _dispatches([r for r in rows if r["Counter_Name"] == counter], "Counter_Value")
            for name, disp in _profiled_dispatches(seq, cfgs, PROFILE_LAUNCHES).items():
                vals[counter][name] = float(np.mean([v for _, v in disp]))
    lines = ["# SQ counters of the attention kernels at 128K context", "",
             "Commands (two passes, one GPU, committed files only):", ""]
    for i, cs in enumerate(SQ_PASSES):
        lines.append(f"    cd /tmp && TMPDIR=/tmp rocprofv3 --pmc {cs} -d <out>/sq{i} -o sq{i} --output-format csv -- "
                     f"python3 /root/repo/bench.py --profile --steps {PROFILE_LAUNCHES}")
    lines += ["", "Per-dispatch averages over each workload's profiled launches (rocprofv3 sums each counter over "
              "the shader engines). Written by `bench.py --write-counters`.", ""]
    lines += [f"kernel_source_sha256_16 ({KERNELS[k][0]}): {kernel_source_hash(k)}" for k in ("f16", "wide")]
    lines += ["", "| counter | " + " | ".join(names) + " |", "|---|" + "---|" * len(names)]
    for counter in sorted(vals):
        lines.append(f"| {counter} | " + " | ".join(f"{vals[counter].get(n, float('nan')):.4g}" for n in names) + " |")

    def ratio(a, b):
        return " | ".join(f"{vals[a][n] / vals[b][n]:.3f}" if vals.get(a, {}).get(n) and vals.get(b, {}).get(n)
                          else "-" for n in names)
    lines += ["", "Derived:", "", "| ratio | " + " | ".join(names) + " |", "|---|" + "---|" * len(names),
              f"| LDS bank-conflict cycles / LDS active cycles | {ratio('SQ_LDS_BANK_CONFLICT', 'SQ_LDS_IDX_ACTIVE')} |",
              f"| LDS active cycles / CU-busy cycles | {ratio('SQ_LDS_IDX_ACTIVE', 'SQ_BUSY_CU_CYCLES')} |",
              f"| MFMA-busy cycles / CU-busy cycles | {ratio('SQ_VALU_MFMA_BUSY_CYCLES', 'SQ_BUSY_CU_CYCLES')} |",
              f"| VALU instructions / LDS instructions | {ratio('SQ_INSTS_VALU', 'SQ_INSTS_LDS')} |",
              f"| VALU instructions / MFMA instructions | {ratio('SQ_INSTS_VALU', 'SQ_INSTS_MFMA')} |"]
    with open(os.path.join(PROFILES, "sq_counters_attn_128k.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("wrote profiles/sq_counters_attn_128k.md")


def write_profiles(bench_kt_dir: str, kt_dir: str, fetch_dir: str, write_dir: str, bench_steps: int):
    """profiles/ summaries. (1) rocprofv3 --kernel-trace --stats of the bench command for the headline workload:
    the --stats line of its kernel and the average of the last `bench_steps` dispatches (the launches bench.py
    times one by one between HIP events, for the roofline). (2) Three rocprofv3 runs of `bench.py --profile
    --steps 20`: per workload the attention dispatches (duration from the kernel trace; FETCH_SIZE and WRITE_SIZE
    per dispatch scaled by what the same counters read for the run's 1 GiB device copies), and the probes."""
    launches = PROFILE_LAUNCHES
    names = ["llama8b_128k_r2"] + [n for n in PROFILE_ALSO if n != "llama8b_128k_r2"]
    cfgs = [workload(n) for n in names]
    trace = _dispatches(_csv_rows(kt_dir, "kernel_trace.csv"))
    fetch = _dispatches(_csv_rows(fetch_dir, "counter_collection.csv"), "Counter_Value")
    write = _dispatches(_csv_rows(write_dir, "counter_collection.csv"), "Counter_Value")

    def copies(seq):  # the three 1 GiB calibration copies (the probes' small read-backs follow them)
        cp = [x for x in seq if "copyBuffer" in x[0]]
        big = max(v for _, v in cp)
        return [x for x in cp if x[1] > 0.5 * big][-3:]

    tokens = {c.name: sum(c.lengths) for c in cfgs}  # (the profiled workloads have fixed lengths)

    def per_workload(seq):
        return _profiled_dispatches(seq, cfgs, launches)
    kt, fe, wr = per_workload(trace), per_workload(fetch), per_workload(write)
    fscale = 1048576.0 / np.mean([v for _, v in copies(fetch)])
    wscale = 1048576.0 / np.mean([v for _, v in copies(write)])
    cmd_kt = ("cd /tmp && TMPDIR=/tmp rocprofv3 --kernel-trace --stats -d <out>/kt -o kt --output-format csv -- "
              f"python3 /root/repo/bench.py --profile --steps {launches}")
    lines = ["# rocprofv3 kernel statistics: decode attention kernels and measurement probes", "",
             "Command (one GPU, committed files only):", "", "    " + cmd_kt, "",
             f"bench.py --profile launches every layer copy of each workload once (setup), keeps the workload running "
             f"for 1 s (the GPU clocks settle), then times {launches} launches rotating over >= 1 GiB of layer copies "
             "(the code stream comes from HBM; each launch between two HIP events, as bench.py times them); then three "
             "1 GiB device copies and the two probes. Summary written by `bench.py --write-profiles`.", "",
             "| workload | kernel | source sha256/16 | dispatches | average us | min us | max us |",
             "|---|---|---|---|---|---|---|"]
    for c in cfgs:
        d = np.array([v for _, v in kt[c.name]]) * 1e-3
        lines.append(f"| {c.name} | {kernel_label(c)} | {kernel_source_hash(kernel_kind(c))} | {len(d)} | "
                     f"{d.mean():.2f} | {d.min():.2f} | {d.max():.2f} |")
    probe_kernels = ("read_stream_kernel", "lds_gather_kernel", "lds_bin_add_kernel")
    probes = [(n, v) for n, v in trace if any(k in n for k in probe_kernels)]
    lines += ["", "| probe | dispatches | average us | what it measures |", "|---|---|---|---|"]
    for key, what in (("read_stream_kernel", "1 GiB streaming read: HBM read rate = 1 GiB / duration"),
                      ("lds_gather_kernel", "1024 WGs x 8 waves x 256 x 16 random 16-byte LDS gathers (1 KiB per "
                                            "wave instruction): gather ceiling = bytes / duration"),
                      ("lds_bin_add_kernel", "1024 WGs x 8 waves x 64 x 84 random 64-bit LDS adds (wave "
                                             "instructions): add ceiling = instructions / duration")):
        d = np.array([v for n, v in probes if key in n]) * 1e-3
        if d.size:
            lines.append(f"| {key} | {len(d)} | {d.mean():.2f} | {what} |")
    # (1) the bench command itself
    prim = workloads.CONFIGS["llama8b_128k_r2"]
    label = kernel_label(prim)
    stats = [r for r in _csv_rows(bench_kt_dir, "kernel_stats.csv") if f"attn_f16_kernel<{prim.n_residuals}>" in r["Name"]]
    btrace = [v for n, v in _dispatches(_csv_rows(bench_kt_dir, "kernel_trace.csv"))
              if f"attn_f16_kernel<{prim.n_residuals}>" in n]
    region = np.array(btrace[-2 * bench_steps:-bench_steps]) * 1e-3
    alone = np.array(btrace[-bench_steps:]) * 1e-3
    cmd_b = ("cd /tmp && TMPDIR=/tmp rocprofv3 --kernel-trace --stats -d <out>/bench -o bench --output-format csv -- "
             f"python3 /root/repo/bench.py --also '' --no-graph --no-cpu-baseline --steps {bench_steps}")
    head = ["# rocprofv3 kernel statistics: decode attention kernels and measurement probes", "",
            f"## The bench command ({prim.name}, {label})", "", "    " + cmd_b, ""]
    if stats:
        r = stats[0]
        head += [f"--stats (every dispatch of {label} in the run: setup, 1 s of clock settling, warmup, the "
                 f"{bench_steps} back-to-back steps and the {bench_steps} event-timed launches): "
                 f"{r['Calls']} calls, average {float(r['AverageNs']) * 1e-3:.2f} us, "
                 f"min {float(r['MinNs']) * 1e-3:.2f} us, max {float(r['MaxNs']) * 1e-3:.2f} us.", ""]
    head += [f"The {len(region)} dispatches of the timed region (back-to-back steps; their average is the "
             f"kernel duration behind the roofline): average {region.mean():.2f} us, min {region.min():.2f} us, "
             f"max {region.max():.2f} us.", "",
             f"The last {len(alone)} dispatches (each launch alone between two HIP events, us_per_launch_isolated): "
             f"average {alone.mean():.2f} us, min {alone.min():.2f} us, max {alone.max():.2f} us.", "",
             "## Per workload (bench.py --profile)", ""]
    lines = head + lines[2:]
    with open(os.path.join(PROFILES, "attn_kernels_128k.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    for c in cfgs:
        algo = algorithmic_bytes(c, tokens[c.name])["codes"]
        fk = float(np.mean([v for _, v in fe[c.name]]))
        wk = float(np.mean([v for _, v in wr[c.name]]))
        hbm = (fk * fscale + wk * wscale) * 1024
        txt = [f"# HBM traffic of {kernel_label(c)} on {c.name}, per dispatch", "",
               "Commands (two passes, one counter each; committed files only):", "",
               "    cd /tmp && TMPDIR=/tmp rocprofv3 --pmc FETCH_SIZE -d <out>/fetch -o fetch --output-format csv -- "
               f"python3 /root/repo/bench.py --profile --steps {launches}",
               "    cd /tmp && TMPDIR=/tmp rocprofv3 --pmc WRITE_SIZE -d <out>/write -o write --output-format csv -- "
               f"python3 /root/repo/bench.py --profile --steps {launches}", "",
               "Calibration: the same runs end with three device copies of exactly 1 GiB; FETCH_SIZE is scaled by "
               f"{fscale:.4f} and WRITE_SIZE by {wscale:.4f} so that each reads 1048576 KiB for them.", "",
               f"kernel_source_sha256_16: {kernel_source_hash(kernel_kind(c))}",
               f"dispatches: {len(fe[c.name])}",
               f"fetch_kib_per_dispatch: {fk:.1f}", f"write_kib_per_dispatch: {wk:.1f}",
               f"fetch_scale: {fscale:.4f}", f"write_scale: {wscale:.4f}",
               f"hbm_bytes_per_launch: {hbm:.0f}", f"algorithmic_code_bytes_per_launch: {algo}",
               f"traffic_over_algorithmic: {hbm / algo:.3f}"]
        with open(os.path.join(PROFILES, f"traffic_attn_decode_{c.name}.txt"), "w") as f:
            f.write("\n".join(txt) + "\n")
    print(f"wrote profiles for {', '.join(names)}")


def workload(name: str):
    return workloads.CONFIGS[name] if name in workloads.CONFIGS else workloads.PAGES_CONFIGS[name]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="llama8b_128k_r2", help="primary workload (value, roofline)")
    ap.add_argument("--also", default="llama8b_128k_r1,llama8b_32k_r1,ragged16_r2,pages_g64_r11_128k,"
                                      "pages_g64_r21_128k,llama8b_8k_r2",
                    help="comma list of extra workloads reported in variants")
    ap.add_argument("--layers", type=int, default=0, help="distinct layer buffers to rotate (0: >= 1 GiB)")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--check", action="store_true", help="compare layer 0 with the oracle")
    ap.add_argument("--profile", action="store_true",
                    help="no timing: a few launches of --config and --also workloads plus a 1 GiB copy, for rocprofv3")
    ap.add_argument("--write-profiles", nargs=4, metavar=("BENCH_KT_DIR", "KT_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="no GPU: write the profiles/ summaries from the csv output of rocprofv3 runs: --kernel-trace "
                         "--stats of `bench.py --also '' --no-graph --no-cpu-baseline --steps K` (K = --steps), and "
                         "three runs of bench.py --profile (--kernel-trace --stats, --pmc FETCH_SIZE, --pmc WRITE_SIZE)")
    ap.add_argument("--write-counters", nargs=2, metavar=("SQ0_DIR", "SQ1_DIR"),
                    help="no GPU: write profiles/sq_counters_attn_128k.md from two rocprofv3 --pmc runs of "
                         "bench.py --profile (the two counter sets of SQ_PASSES)")
    args = ap.parse_args()
    if args.write_counters:
        write_counters(args.write_counters)
        return
    if args.write_profiles:
        write_profiles(*args.write_profiles, bench_steps=args.steps)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "bench.py measures one GPU; sharding across GPUs is not implemented", "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.profile:  # a fixed set, in the dispatch order the profile summaries are read in
        names = [args.config] + [s for s in PROFILE_ALSO if s != args.config]
        profile_run(names, max(args.steps, 1))
        return
    cfg = workloads.CONFIGS[args.config]
    probes = {"hbm_read_stream": read_stream_probe(), "lds_random_gather": lds_gather_probe(),
              "lds_bin_add": lds_bin_add_probe()}
    prim, base = run_config(cfg, args.steps, args.warmup, args.layers, not args.no_graph, args.check, probes)
    variants = {cfg.name: prim}
    for name in [s for s in args.also.split(",") if s and s != cfg.name]:
        variants[name], _ = run_config(workload(name), args.steps, args.warmup, args.layers, not args.no_graph,
                                       args.check, probes)
        if name in PAGES_CONTEXT:
            variants[name]["pages_context"] = PAGES_CONTEXT[name]

    achieved = prim["bytes"]["codes"] / (prim["ms_per_step"] * 1e-3) * 1e-9
    traffic = read_traffic(cfg)
    line = {
        "metric": "decode-attn KV tokens/s per layer at 128K ctx, 1/2-bit; % of HBM roofline",
        "value": prim["kv_tokens_per_s_per_layer"],
        "unit": "KV tokens/s per layer",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": prim["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16 (fp32 accumulate)" if cfg.dtype == "float16" else "f32",
        "data": "synthetic (seeded workloads generator; uniform code indices, N(0,0.25) codebooks)",
        "config": {"workload": cfg.name, "batch": cfg.batch, "kv_heads": cfg.n_kv_heads, "q_heads": cfg.n_q_heads,
                   "head_dim": cfg.head_dim, "context": prim["tokens"], "residuals": cfg.n_residuals,
                   "groups": cfg.n_groups, "codes": cfg.n_codes, "layers_rotated": prim["layers_rotated"]},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                     "kernel": f"{kernel_label(cfg)} (fused decode attention, one launch per layer)",
                     "algorithmic_bytes_per_launch": prim["bytes"]["codes"]},
        "variants": variants,
        "probes": probes,
        "kernel_source_sha256_16": {kind: kernel_source_hash(kind) for kind in KERNELS},
    }
    line["steps"] = step_kernels_timing(probes)
    line["codebook_tools"] = codebook_tools_timing()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, base)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
