#!/usr/bin/env python3
"""Benchmark of the routed, block-quantized MoE layer on one MI355X.

A step is one pass of the whole layer (router, top-k + softmax, permutation/union, expert FFNs,
combine + shared expert) over one batch of seeded synthetic input, as ``moe_layer`` calls:

  decode1 (default): 1 token, H 2048, 256 experts top-8 + shared (I 512), 4-bit experts. The layer
      is replicated 48 times at distinct HBM addresses (all 256 experts of each copy resident) and
      one step is 48 sequential ``moe_layer`` calls, one per copy, so every call streams its
      experts from HBM rather than from the 256 MB Infinity Cache. The step is captured once as a
      HIP graph and replayed (``--eager`` launches every call from Python instead).
  verify4: the same with 4 tokens and 8-bit experts.
  stack48: 48 distinct layers of 512 experts top-10, 2-bit experts, 1 token (36 GB resident).
  prefill8k: one 8192-token chunk through one layer (256 experts, 4-bit, shared expert).

value = MoE-layer tokens/s = (layer calls x tokens per call) / time, inputs resident in HBM.
The JSON line also carries the roofline of the dominant kernel stage (expert weight bytes per
launch over its HIP-event-timed duration for decode; expert FLOPs for prefill) and the fp64 CPU
oracle timed on a bounded sample of the same workload on this host.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
import quantized_expert_ffn_moe_amd as moe  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_F16_PEAK_TFS = 2516.6     # MI355X dense fp16/bf16 MFMA, TFLOP/s (256 CU x 4096 flop/clk x 2.4 GHz)
REPLICAS = 48


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def expert_weight_bytes(spec, n_routed: int) -> int:
    """Packed codes + fp16 scales of n_routed routed experts plus the shared expert."""
    b = n_routed * spec.expert_bytes()
    if spec.Is:
        b += spec.expert_bytes(spec.Is)
    return b


def upload(spec, d):
    return moe.DeviceLayer.from_host(moe.LayerDesc.from_spec(spec), d)


def clone_layer(L: moe.DeviceLayer) -> moe.DeviceLayer:
    def c(p):
        return None if p is None else (p[0].clone(), p[1].clone())
    m = L.mats
    return moe.DeviceLayer(L.desc, L.w_router.clone(), None if L.router_bias is None else L.router_bias.clone(),
                           c(m["gate"]), c(m["up"]), c(m["down"]), c(m["sh_gate"]), c(m["sh_up"]), c(m["sh_down"]))


def dev_x(x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda()


# Kernel sources behind each measured stage: a recorded HBM-traffic figure (profiles/*_traffic.md,
# from rocprofv3 FETCH_SIZE / WRITE_SIZE runs) is reported only while these files are unchanged.
STAGE_SOURCES = {
    "decode": ["csrc/decode.hip", "csrc/common.h", "csrc/kernels.h"],
    "prefill": ["csrc/prefill.hip", "csrc/common.h", "csrc/kernels.h"],
}


def sources_digest(stage: str) -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in STAGE_SOURCES[stage]:
        with open(os.path.join(ROOT, "quantized_expert_ffn_moe_amd", rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(workload: str, stage: str):
    """HBM bytes per launch recorded in profiles/<workload>_traffic.md, or None when absent or when
    the kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "%s_traffic.md" % workload)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            line = line.strip().strip("`")
            if "=" in line and line.split("=")[0].strip() in ("traffic_bytes_per_launch", "sources_sha256"):
                k, v = line.split("=", 1)
                vals[k.strip()] = v.strip()
    if vals.get("sources_sha256") != sources_digest(stage) or "traffic_bytes_per_launch" not in vals:
        return None
    return int(float(vals["traffic_bytes_per_launch"]))


def calibrate_copy(mib: int = 256, reps: int = 3):
    """Plain device-to-device copies of a known size, for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    src = torch.empty(mib << 20, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log("copy calibration: %d x %d MiB device-to-device" % (reps, mib))


def capture(fn_list):
    """One HIP graph holding the launches of fn_list in order (the library launches on torch's
    current stream, which is the capture stream inside torch.cuda.graph)."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in fn_list:
            f()
    torch.cuda.synchronize()
    return g


def time_calls(fn_list, warmup: int, reps: int, graph: bool = False) -> float:
    """Average duration (ms) of one launch from a list of zero-arg launches, played back to back
    reps times between two HIP events on torch's current stream (the stream the library uses);
    with graph=True the list is captured once and the graph replayed."""
    for _ in range(warmup):
        for f in fn_list:
            f()
    torch.cuda.synchronize()
    g = capture(fn_list) if graph else None
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        if g is not None:
            g.replay()
        else:
            for f in fn_list:
                f()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / (reps * len(fn_list))


def decode_workload(name: str, steps: int, warmup: int, graph: bool = True):
    spec = synth.CONFIGS[name]
    layers = []
    xs = []
    t0 = time.time()
    if name == "stack48":
        for l in range(spec.layers):
            d = synth.make_layer(spec, layer=l)
            layers.append(upload(spec, d))
            xs.append(dev_x(d["x"]))
            log("generated layer %d/%d (%.0f s)" % (l + 1, spec.layers, time.time() - t0))
    else:
        d = synth.make_layer(spec)
        base = upload(spec, d)
        layers = [base] + [clone_layer(base) for _ in range(REPLICAS - 1)]
        xs = [dev_x(d["x"])] * REPLICAS
    torch.cuda.synchronize()
    log("%s: %d resident layer copies ready in %.1f s" % (name, len(layers), time.time() - t0))
    T = spec.T
    ws = moe.Workspace()
    out = torch.empty((T, spec.H), dtype=torch.float32, device="cuda")
    ids = [torch.empty((T, spec.k), dtype=torch.int32, device="cuda") for _ in layers]
    calls = [lambda L=L, x=x, i=i: moe.moe_layer(L, x, out=out, ids=i, ws=ws) for L, x, i in zip(layers, xs, ids)]

    def step():
        for c in calls:
            c()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # one step (all layer calls) captured as a HIP graph and replayed: the launches of a decode
    # step are issued once, as a serving loop would
    g = capture(calls) if graph else None
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        if g is not None:
            g.replay()
        else:
            step()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b)
    ms_per_step = ms / steps
    value = len(layers) * T * steps / (ms / 1e3)

    # dominant stage: the decode expert FFNs (moe_experts_decode), timed per launch with HIP events
    nU = [len(set(i.cpu().numpy().ravel().tolist())) for i in ids]
    ysh = torch.empty((T, spec.H), dtype=torch.float32, device="cuda")
    ypairs = torch.empty((T * spec.k, spec.H), dtype=torch.float32, device="cuda")
    ews = moe.Workspace()
    ecalls = [lambda L=L, x=x, i=i: moe.moe_experts_decode(L, x, i, y_pairs=ypairs, y_shared=ysh, ws=ews)
              for L, x, i in zip(layers, xs, ids)]
    avg_ms = time_calls(ecalls, 2, max(3, steps), graph=graph)
    bytes_per_launch = float(np.mean([expert_weight_bytes(spec, u) for u in nU]))
    achieved = bytes_per_launch / (avg_ms / 1e3) / 1e9
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": recorded_traffic(name, "decode"),
            "kernel": "moe_experts_decode (k_dec_gateup + k_dec_down), back-to-back over the resident copies"
                      + (" (one HIP graph)" if graph else ""),
            "bytes_per_launch": int(bytes_per_launch), "avg_launch_us": round(avg_ms * 1e3, 2),
            "distinct_experts_per_call": float(np.mean(nU))}
    cfg = {"workload": name, "tokens_per_call": T, "hidden": spec.H, "experts": spec.E, "top_k": spec.k,
           "inter": spec.I, "shared_inter": spec.Is, "format": synth.FMT_NAMES[spec.fmt],
           "layer_calls_per_step": len(layers), "resident_layers": len(layers),
           "launch": "hip_graph" if graph else "eager"}
    del layers, calls, ecalls
    torch.cuda.empty_cache()
    return value, ms_per_step, roof, cfg


def prefill_workload(steps: int, warmup: int):
    spec = synth.CONFIGS["prefill8k"]
    t0 = time.time()
    d = synth.make_layer(spec)
    L = upload(spec, d)
    L.pack_prefill_codes()   # the grouped GEMMs' copy of the codes, made once like the weights (not timed)
    x = dev_x(d["x"])
    torch.cuda.synchronize()
    log("prefill8k ready in %.1f s" % (time.time() - t0))
    T = spec.T
    ws = moe.Workspace()
    out = torch.empty((T, spec.H), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, spec.k), dtype=torch.int32, device="cuda")
    for _ in range(warmup):
        moe.moe_layer(L, x, out=out, ids=ids, ws=ws)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        moe.moe_layer(L, x, out=out, ids=ids, ws=ws)
    b.record()
    torch.cuda.synchronize()
    ms_per_step = a.elapsed_time(b) / steps
    value = T / (ms_per_step / 1e3)
    # expert stage on its own, in the form the layer runs it (fp16 output rows)
    offsets, perm, inv = moe.moe_permute(L, ids)
    y_sorted = torch.empty((T * spec.k, spec.H), dtype=torch.float16, device="cuda")
    y_sh = torch.empty((T, spec.H), dtype=torch.float16, device="cuda")
    pws = moe.Workspace()
    avg_ms = time_calls([lambda: moe.moe_experts_prefill(L, x, offsets, perm, y_sorted=y_sorted, y_shared=y_sh,
                                                         ws=pws, half=True)], 2, max(3, steps))
    flops = 6.0 * spec.H * spec.I * (T * spec.k) + 6.0 * spec.H * spec.Is * T
    achieved = flops / (avg_ms / 1e3) / 1e12
    roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_F16_PEAK_TFS, "unit": "TFLOP/s",
            "frac": round(achieved / MFMA_F16_PEAK_TFS, 4), "traffic": recorded_traffic("prefill8k", "prefill"),
            "kernel": "moe_experts_prefill_f16 (k_x_to_f16 with the tile list + k_grouped_gemm gate/up + k_grouped_gemm down)",
            "flops_per_launch": flops, "avg_launch_us": round(avg_ms * 1e3, 1)}
    return {"metric": "MoE-layer tokens/s (8192-token prefill chunk)", "value": round(value, 1),
            "unit": "tokens/s", "dtype": "f16", "ms_per_step": round(ms_per_step, 4),
            "roofline": roof,
            "config": {"workload": "prefill8k", "tokens_per_call": T, "hidden": spec.H, "experts": spec.E,
                       "top_k": spec.k, "inter": spec.I, "shared_inter": spec.Is,
                       "format": synth.FMT_NAMES[spec.fmt],
                       "codes": "packed copy for the grouped GEMMs (moe_pack_prefill_codes, made at setup)"}}


def kv_workload(reps: int = 20):
    """The int8 block-32 KV codec on a cache of 131072 positions x 512 values (bf16 in): encode of
    the whole cache, and the sparse gather of 16 queries x 2048 positions (exact fp32 rows out).
    Both are HBM streams: bytes moved per launch over the HIP-event-timed duration."""
    n_rows, D, n_idx = 131072, 512, 16 * 2048
    g = torch.Generator(device="cuda").manual_seed(7)
    x = torch.randn((n_rows, D), generator=g, device="cuda").to(torch.bfloat16)
    codes = torch.empty((n_rows, D), dtype=torch.int8, device="cuda")
    scales = torch.empty((n_rows, D // 32), dtype=torch.int16, device="cuda")
    idx = torch.randint(0, n_rows, (n_idx,), generator=g, device="cuda", dtype=torch.int32)
    out = torch.empty((n_idx, D), dtype=torch.float32, device="cuda")
    enc_ms = time_calls([lambda: moe.moe_kv_encode(x, codes, scales)], 3, reps)
    gat_ms = time_calls([lambda: moe.moe_kv_gather(codes, scales, idx, out=out)], 3, reps)
    enc_bytes = n_rows * D * 2 + n_rows * D + n_rows * (D // 32) * 2
    gat_bytes = n_idx * 4 + n_idx * D + n_idx * (D // 32) * 2 + n_idx * D * 4

    def roof(nbytes, ms, kernel):
        a = nbytes / (ms / 1e3) / 1e9
        return {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(a / HBM_PEAK_GBS, 4), "traffic": None, "kernel": kernel,
                "bytes_per_launch": int(nbytes), "avg_launch_us": round(ms * 1e3, 2)}
    return {"workload": "int8 block-32 KV cache, 131072 positions x 512, gather 16 x 2048 positions",
            "encode": roof(enc_bytes, enc_ms, "k_kv_encode"), "gather": roof(gat_bytes, gat_ms, "k_kv_gather")}


def sweep_tokens(reps: int = 20):
    """Mid-size batches: moe_layer time per call for T = 1 .. 8192 tokens on the prefill8k layer
    (hidden 2048, 256 experts top-8 + shared, 4-bit), each T captured as a HIP graph of 10 calls and
    replayed. moe_layer's default regime switch is timed at every T; for T <= 8 also both regimes
    forced through the descriptor's decode_max_tokens (8: decode kernels, 1: grouped GEMMs)."""
    spec = synth.CONFIGS["prefill8k"]
    d = synth.make_layer(spec)
    L = upload(spec, d)
    L.pack_prefill_codes()   # as in the prefill8k measurement

    def with_desc(dmt):
        m = L.mats
        Lx = moe.DeviceLayer(moe.LayerDesc.from_spec(spec, dmt), L.w_router, L.router_bias, m["gate"], m["up"],
                             m["down"], m["sh_gate"], m["sh_up"], m["sh_down"])
        Lx.prefill_codes, Lx.c.prefill_codes = L.prefill_codes, L.c.prefill_codes
        return Lx
    Ld, Lg = with_desc(8), with_desc(1)
    xs_all = dev_x(d["x"])
    rows = []
    for T in [1, 2, 3, 4, 5, 6, 7, 8, 12, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096, 8192]:
        x = xs_all[:T].contiguous()
        out = torch.empty((T, spec.H), dtype=torch.float32, device="cuda")

        def timed(layer):
            ws = moe.Workspace()
            return time_calls([lambda: moe.moe_layer(layer, x, out=out, ws=ws)] * 10, 2, reps, graph=True)
        row = {"T": T, "us_per_call": round(timed(L) * 1e3, 2)}
        row["tokens_per_s"] = round(T / (row["us_per_call"] / 1e6), 1)
        if T <= 8:
            row["decode_kernels_us"] = round(timed(Ld) * 1e3, 2)
            row["grouped_gemm_us"] = round(timed(Lg) * 1e3, 2)
        rows.append(row)
        log("T=%d: %s" % (T, row))
    return rows


def host_cpu():
    """CPU model and logical core count of this host (for the CPU-baseline records)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, os.cpu_count() or 0


def cpu_baseline(name: str, budget_s: float = 6.0):
    """The fp64 oracle, single-threaded, on a bounded sample of the same workload: the same layer
    and the same input tokens the GPU run uses (layer 0 for the 48-layer stack, whose layers all
    have the same shape; the first tokens of the 8192-token chunk for prefill, whose cost is
    linear in tokens, so tokens/s of the sample is the chunk's rate)."""
    import oracle
    spec = synth.CONFIGS[name]
    d = synth.make_layer(spec, layer=0)
    O = oracle.Layer.from_synth(spec, d)
    xs = d["x"]
    n = 0
    t0 = time.perf_counter()
    while True:
        O.token(xs[n % xs.shape[0]])
        n += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    model, nproc = host_cpu()
    what = {"prefill8k": "the first %d of the 8192 tokens of the chunk (extrapolated: cost is linear in tokens)" % n,
            "stack48": "%d tokens through layer 0 of the stack (every layer has the same shape)" % n}.get(
        name, "%d tokens (the GPU run's own input%s) through the full layer" % (n, "s, cycled" if spec.T > 1 else ""))
    return {"value": round(n / el, 3), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": "%s: router, top-k, experts, combine in fp64 on 1 thread, %.1f s" % (what, el),
            "host_nproc": nproc, "host_cpu": model, "workload": name}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="decode1", choices=["decode1", "verify4", "stack48", "prefill8k"])
    ap.add_argument("--no-prefill", action="store_true", help="skip the secondary 8K prefill measurement")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kv", action="store_true", help="skip the secondary KV-codec measurement")
    ap.add_argument("--no-other-decode", action="store_true",
                    help="with the default decode1 workload, skip the secondary verify4 and stack48 lines")
    ap.add_argument("--eager", action="store_true",
                    help="launch every decode call from Python instead of replaying one captured HIP graph per step")
    ap.add_argument("--sweep-tokens", action="store_true",
                    help="print moe_layer time per call for T = 1 .. 8192 (mid-size batches) and exit")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first copy 256 MiB device-to-device 3 times (scale for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (expert parallelism is a design "
              "note); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    moe.lib()
    if args.calibrate_copy:
        calibrate_copy()
    if args.sweep_tokens:
        print(json.dumps({"sweep": "moe_layer time per call vs tokens per call (HIP graph replays)",
                          "layer": "prefill8k shape", "rows": sweep_tokens()}), flush=True)
        return

    others = {}
    if args.workload == "prefill8k":
        r = prefill_workload(args.steps, args.warmup)
        value, ms, roof, cfg, metric = r["value"], r["ms_per_step"], r["roofline"], r["config"], r["metric"]
        secondary = None
    else:
        value, ms, roof, cfg = decode_workload(args.workload, args.steps, args.warmup, graph=not args.eager)
        metric = "MoE-layer tokens/s (decode, %% HBM peak on expert-weight bytes)"
        secondary = None if args.no_prefill else prefill_workload(max(10, args.steps), 3)
        if args.workload == "decode1" and not args.no_other_decode:
            # the other decode workloads as secondary lines of the same run
            for w in ("verify4", "stack48"):
                v2, ms2, roof2, cfg2 = decode_workload(w, max(5, args.steps // 2), 2, graph=not args.eager)
                others[w] = {"metric": "MoE-layer tokens/s (decode, % HBM peak on expert-weight bytes)",
                             "value": round(v2, 1), "unit": "tokens/s", "ms_per_step": round(ms2, 4),
                             "dtype": "f16", "roofline": roof2, "config": cfg2}
    line = {"metric": metric.replace("%%", "%"), "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "f16",
            "data": "synthetic (seeded N(0,0.02) weights quantised to block-32 codes, bf16 N(0,1) activations, "
                    "Zipf-biased router)",
            "config": cfg, "roofline": roof}
    for w, o in others.items():
        line[w] = o
    if secondary is not None:
        line["prefill"] = secondary
    if not args.no_kv and args.workload != "prefill8k":
        line["kv_cache"] = kv_workload()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args.workload)
        if args.workload == "decode1":
            for w in list(others) + ([] if secondary is None else ["prefill8k"]):
                obj = line["prefill"] if w == "prefill8k" else line[w]
                obj["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
