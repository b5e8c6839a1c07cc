#!/usr/bin/env python3
"""Benchmark: CommVQ decode-step attention, KV tokens/s per layer at 128K context (1-bit and 2-bit).

One step = one decode-step attention call for one layer (every row of the hot path: code stream and
unpack, RoPE phases, key scores, split softmax, value reduce, combine) on the Llama-3.1-8B layer shape
(8 KV / 32 q heads, head dim 128, G = 16, N = 256). Steps rotate over `layers` distinct copies of the
layer's codes, codebooks and query (>= 1 GiB in total) so the 256 MB Infinity Cache cannot serve
the code stream. Inputs are synthetic (workloads.make_inputs) and resident in HBM before timing.

Prints one JSON line. The timed region is K steps between two device synchronizations; the
per-launch kernel duration for the roofline comes from HIP events recorded on the launch stream.
cpu_baseline times the fp64 oracle on the host on a bounded sample of the same workload.
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
# per CU); random 16-byte gathers measured at 12.04 clocks per 1 KiB wave instruction (bank conflicts)
LDS_PEAK_TBPS = 256 * 256 * 2.4e9 / 1e12
LDS_GATHER_TBPS = 256 * 1024 / 12.04 * 2.4e9 / 1e12
PROFILES = os.path.join(ROOT, "profiles")
# sources that determine each attention kernel's memory traffic (split sizing, layout, kernel body)
_CSRC = os.path.join(ROOT, "vector_quantized_kv_amd", "csrc")
KERNEL_SOURCES = [os.path.join(_CSRC, f) for f in
                  ("attn.hip", "attn_common.h", "commvq_internal.h", "device_common.h", "api.cpp")]
WIDE_KERNEL_SOURCES = [os.path.join(_CSRC, f) for f in
                       ("attn_wide.hip", "attn_common.h", "commvq_internal.h", "device_common.h", "api.cpp")]
KERNEL_NAME = "attn_kernel"


def kernel_source_hash(sources=None) -> str:
    h = hashlib.sha256()
    for p in sources or KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(config_name: str, sources=None):
    """HBM bytes per launch from the committed rocprofv3 PMC summary, if it matches the current kernels."""
    path = os.path.join(PROFILES, f"traffic_attn_decode_{config_name}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != kernel_source_hash(sources):
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
    return {"value": d_tokens / per_run, "unit": "KV tokens/s per layer", "cores": threads, "kind": "oracle",
            "sample": f"{runs} full decode steps of one layer ({cfg.name}: {d_tokens} tokens x "
                      f"{cfg.n_kv_heads} KV heads), fp64, {threads} host threads; {per_run:.3f} s per step"}


def read_stream_gbps(nbytes: int = 1 << 30, reps: int = 10) -> float:
    """Achievable HBM read rate on this machine: torch.sum over a 1 GiB fp32 tensor (one read pass each)."""
    import torch
    x = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    for _ in range(2):
        x.sum()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        x.sum()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    del x
    return nbytes / (ms * 1e-3) * 1e-9


def profile_run(names, launches: int):
    """Few launches per workload (for rocprofv3), plus a 1 GiB device copy whose FETCH_SIZE / WRITE_SIZE
    calibrate the counters (it reads and writes exactly 1 GiB)."""
    import torch
    import vector_quantized_kv_amd as vq
    for name in names:
        cfg = workload(name)
        d = vq.dims_of(cfg)
        base = workloads.make_inputs(cfg)
        per_layer = algorithmic_bytes(cfg, int(base["total_tokens"]))["total"]
        layers = max(4, int(math.ceil((1 << 30) / per_layer)))
        rope = vq.rope_table(d, int(base["max_len"]))
        Ls = [vq.Layer(d, base if i == 0 else workloads.make_inputs(cfg, seed=cfg.seed + 1000 * i), rope=rope,
                       rope_positions=int(base["max_len"])) for i in range(layers)]
        for i in range(launches):
            Ls[i % layers].attn_decode()
        torch.cuda.synchronize()
        print(f"profile: {name} {launches} launches over {layers} layer copies", flush=True)
        del Ls
        torch.cuda.empty_cache()
    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print("profile: 3 copies of 1 GiB (calibration)", flush=True)


def run_config(cfg, steps: int, warmup: int, layers: int, use_graph: bool, check: bool):
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
    torch.cuda.synchronize()
    check_err = None
    if check:
        import oracle
        got = Ls[0].attn_decode().cpu().numpy().astype(np.float64)
        ref = oracle.run_config(cfg, base, n_threads=min(len(os.sched_getaffinity(0)), 16))
        check_err = float((np.abs(got - ref).max(-1) / np.abs(ref).max(-1)).max())

    stream = torch.cuda.current_stream()
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

    # per-launch kernel duration for the roofline: HIP events on the launch stream around each call
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
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        reps = max(1, steps // layers)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        graph_ms = a.elapsed_time(b) / (reps * layers)

    per_step_ms = total_ms / steps
    print(f"[bench] {cfg.name}: {layers} layers, {launch_ms * 1e3:.1f} us per launch", file=sys.stderr, flush=True)
    L = total
    res = {
        "config": cfg.name, "tokens": L, "layers_rotated": layers, "ms_per_step": per_step_ms,
        "us_per_layer_eager": per_step_ms * 1e3, "us_per_launch": launch_ms * 1e3,
        "us_per_layer_graph": None if graph_ms is None else graph_ms * 1e3,
        "kv_tokens_per_s_per_layer": L / (per_step_ms * 1e-3),
        "code_stream_GBps": per_layer["codes"] / (launch_ms * 1e-3) * 1e-9,
        "compulsory_GBps": per_layer["total"] / (launch_ms * 1e-3) * 1e-9,
        "pct_hbm_peak_code_stream": 100.0 * per_layer["codes"] / (launch_ms * 1e-3) * 1e-9 / HBM_PEAK_GBPS,
        "bytes": per_layer, "max_row_rel_err_vs_oracle": check_err,
    }
    # Every token gathers, per residual and group, its codeword row from LDS for keys and again for values
    # (16 bytes in the byte layout, 128 in the bit-packed one, at fp16): that LDS stream is what bounds both
    # kernels. The whole launch, fixed costs included, is counted against it.
    gathered = 2 * cfg.n_kv_heads * L * cfg.n_residuals * cfg.n_groups * cfg.group_dim * \
        (2 if cfg.dtype == "float16" else 4)
    tbps = gathered / (launch_ms * 1e-3) * 1e-12
    res["lds_roofline"] = {"bound": "lds", "gathered_bytes_per_launch": gathered, "achieved": tbps,
                           "unit": "TB/s", "peak": LDS_PEAK_TBPS, "frac": tbps / LDS_PEAK_TBPS,
                           "random_gather_ceiling": LDS_GATHER_TBPS,
                           "frac_of_random_gather_ceiling": tbps / LDS_GATHER_TBPS}
    if cfg.packed:
        res["hbm_traffic_bytes_per_launch"] = read_traffic(cfg.name, WIDE_KERNEL_SOURCES)
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
        # the library is built without packed-fp32 instructions, so its fp32 VALU peak is half the published
        # 157.3 TFLOP/s: 256 CUs x 4 SIMDs x 16 lanes x 2 flops (FMA) x 2.4 GHz = 78.6 TFLOP/s
        "encode_greedy": {"ms": t_enc * 1e3, "tokens_per_s": n / t_enc, "bound": "alu",
                          "achieved_tflops": enc_flops / t_enc * 1e-12, "peak_tflops": 78.6,
                          "frac": enc_flops / t_enc * 1e-12 / 78.6},
        "codebook_update": {"ms": t_upd * 1e3, "tokens_per_s": n / t_upd},
        "encode_greedy_bit_packed_r21": {"ms": t_encb * 1e3, "tokens_per_s": n / t_encb, "bound": "alu",
                                         "achieved_tflops": encb_flops / t_encb * 1e-12, "peak_tflops": 78.6,
                                         "frac": encb_flops / t_encb * 1e-12 / 78.6},
        "codebook_update_bit_packed_r21": {"ms": t_updb * 1e3, "tokens_per_s": n / t_updb},
    }


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


def workload(name: str):
    return workloads.CONFIGS[name] if name in workloads.CONFIGS else workloads.PAGES_CONFIGS[name]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="llama8b_128k_r2", help="primary workload (value, roofline)")
    ap.add_argument("--also", default="llama8b_128k_r1,pages_g64_r11_128k,pages_g64_r21_128k,llama8b_8k_r2",
                    help="comma list of extra workloads reported in variants")
    ap.add_argument("--layers", type=int, default=0, help="distinct layer buffers to rotate (0: >= 1 GiB)")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--check", action="store_true", help="compare layer 0 with the oracle")
    ap.add_argument("--profile", action="store_true",
                    help="no timing: a few launches of --config and --also workloads plus a 1 GiB copy, for rocprofv3")
    args = ap.parse_args()

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
    prim, base = run_config(cfg, args.steps, args.warmup, args.layers, not args.no_graph, args.check)
    variants = {cfg.name: prim}
    for name in [s for s in args.also.split(",") if s and s != cfg.name]:
        variants[name], _ = run_config(workload(name), args.steps, args.warmup, args.layers, not args.no_graph,
                                       args.check)
        if name in PAGES_CONTEXT:
            variants[name]["pages_context"] = PAGES_CONTEXT[name]

    achieved = prim["bytes"]["codes"] / (prim["us_per_launch"] * 1e-6) * 1e-9
    traffic = read_traffic(cfg.name)
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
                     "kernel": f"{KERNEL_NAME} (fused decode attention, one launch per layer)",
                     "algorithmic_bytes_per_launch": prim["bytes"]["codes"]},
        "variants": variants,
        "hbm_read_stream_GBps": read_stream_gbps(),
        "kernel_source_sha256_16": kernel_source_hash(),
        "wide_kernel_source_sha256_16": kernel_source_hash(WIDE_KERNEL_SOURCES),
    }
    line["codebook_tools"] = codebook_tools_timing()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, base)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
