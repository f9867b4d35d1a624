"""Benchmark: microseconds per packed-MoE layer at T=1 on the 30B-A3B expert shape
(E=128, H=2048, I=768, top-8, FP4 E2M1, group 32), with achieved HBM GB/s over the bytes
of the active experts' packed weights and scales, against the 8 TB/s MI355X peak.

One step = one token through a stack of `--layers` distinct layer weight sets (48 by
default, about 1 GB of active expert bytes per step, four times the 256 MB last-level
cache), each layer = routing from fp32 logits + gate_up + SiLU*up + down + top-k combine
in one `moe_fp4_layer` call.  The layers are captured once into a graph; the timed region
replays it K times between events on the capturing stream.  Inputs (weights, scales,
activations, logits) are synthetic and already resident in device memory.

Prints one JSON line (see the repository docs for the fields).  `--gpus` above 1 exits:
this benchmark is single-GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs per MoE layer at T=1 and achieved HBM GB/s vs peak (Qwen3-30B-A3B shape)"
HBM_PEAK_GBPS = 8000.0
SHAPE = dict(T=1, E=128, H=2048, I=768, k=8, group=32)


def active_bytes(H, I, G, k):
    per_expert = (H // 2) * (2 * I) + (H // G) * (2 * I) * 2 + (I // 2) * H + (I // G) * H * 2
    return k * per_expert, per_expert


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "dequant_gemv_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def build_workload(layers: int, seed: int = 0, device="cuda"):
    """Layer weight sets drawn on the device: packed bytes uniform over 0..255 (every
    nibble uniform), scales U(0.002, 0.01) rounded to bf16, x ~ N(0,1) in bf16, logits
    ~ N(0,1) fp32, one set per layer."""
    import torch
    T, E, H, I, G = SHAPE["T"], SHAPE["E"], SHAPE["H"], SHAPE["I"], SHAPE["group"]
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = []
    for _ in range(layers):
        L = dict(
            w_gu=torch.randint(0, 256, (E, H // 2, 2 * I), dtype=torch.uint8, device=device,
                               generator=g),
            s_gu=(torch.rand((E, H // G, 2 * I), device=device, generator=g) * 0.008 + 0.002
                  ).to(torch.bfloat16),
            w_d=torch.randint(0, 256, (E, I // 2, H), dtype=torch.uint8, device=device,
                              generator=g),
            s_d=(torch.rand((E, I // G, H), device=device, generator=g) * 0.008 + 0.002
                 ).to(torch.bfloat16),
            logits=torch.randn((T, E), device=device, generator=g, dtype=torch.float32),
        )
        out.append(L)
    x = torch.randn((T, H), device=device, generator=g).to(torch.bfloat16)
    return x, out


def cpu_baseline(budget_s: float = 12.0):
    """The float64 oracle on the same layer shape, single-threaded BLAS, for a bounded
    number of layers (about `budget_s` seconds).  Returns µs per layer."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import moe_oracle as O
    from workloads import synth as S
    cfg = S.Q30
    layers, t_total, n = 0, 0.0, 0
    with threadpool_limits(limits=1):
        seed = 0
        while t_total < budget_s and n < 64:
            ids_needed = O.topk_route(S.moe_layer_logits(cfg, seed), cfg.k)[0]
            L = S.make_moe_layer(cfg, seed, experts=np.unique(ids_needed))
            t0 = time.perf_counter()
            O.moe_layer(L.x, L.logits, cfg.k, L.w_gu, L.s_gu, L.w_d, L.s_d, cfg.group, cfg.fmt)
            t_total += time.perf_counter() - t0
            n += 1
            seed += 1
    return {"value": t_total / n * 1e6, "unit": "us/layer", "cores": 1, "kind": "oracle",
            "sample": f"{n} Q30 T=1 layers (route + 8 experts + combine), float64 numpy, "
                      f"one BLAS thread, {t_total:.1f} s total"}


def read_traffic(kernel: str):
    """HBM traffic per launch from the committed rocprofv3 counter summary, or None when
    the kernel sources changed since the counters were taken."""
    p = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
    except Exception:
        return None
    e = d.get(kernel)
    if not e or e.get("source_hash") != kernel_source_hash():
        return None
    return e.get("hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=48)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--path", choices=["auto", "unfused"], default="auto")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES bytes (3 times); "
                         "used to scale rocprofv3 FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the path "
              "is single-GPU; see the sharding notes in the design document)", file=sys.stderr)
        sys.exit(2)

    import torch

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        n = args.copy_calibration
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize(dev)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize(dev)
        print(json.dumps({"copy_calibration_bytes": n}))
        return

    from dequant_gemv_amd import binding as B
    T, E, H, I, k, G = (SHAPE[s] for s in ("T", "E", "H", "I", "k", "group"))
    flags = B.PATH_NO_FUSED if args.path == "unfused" else 0
    x, layers = build_workload(args.layers, device=dev)
    ws = B.moe_workspace(T, H, I, E, k, dev)
    outs = [torch.empty((T, H), dtype=torch.bfloat16, device=dev) for _ in layers]

    def one_pass():
        for L, o in zip(layers, outs):
            B.moe_fp4_layer(x, L["logits"], k, L["w_gu"], L["s_gu"], L["w_d"], L["s_d"], G,
                            B.FMT_FP4_E2M1, out=o, workspace=ws, flags=flags)

    stream = torch.cuda.Stream(device=dev)
    stream.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(stream):
        one_pass()  # eager warm-up on the capture stream
    stream.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        one_pass()
    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            graph.replay()
    stream.synchronize()
    torch.cuda.synchronize(dev)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(args.steps):
            graph.replay()
        e1.record(stream)
    e1.synchronize()
    torch.cuda.synchronize(dev)
    ms = e0.elapsed_time(e1)
    ms_per_step = ms / args.steps
    us_per_layer = ms_per_step * 1000.0 / args.layers

    # context only: events right before and after each eager layer call (includes the
    # host launch overhead that the graph replay hides)
    per = []
    with torch.cuda.stream(stream):
        for rep in range(3):
            for L, o in zip(layers, outs):
                a0 = torch.cuda.Event(enable_timing=True)
                a1 = torch.cuda.Event(enable_timing=True)
                a0.record(stream)
                B.moe_fp4_layer(x, L["logits"], k, L["w_gu"], L["s_gu"], L["w_d"], L["s_d"], G,
                                B.FMT_FP4_E2M1, out=o, workspace=ws, flags=flags)
                a1.record(stream)
                per.append((a0, a1))
    stream.synchronize()
    eager_us = sorted(a0.elapsed_time(a1) * 1000.0 for a0, a1 in per)[len(per) // 2]

    abytes, _ = active_bytes(H, I, G, k)
    fused = args.path == "auto" and T == 1
    launches_per_layer = 1 if fused else 3
    gbps = abytes / (us_per_layer * 1e-6) / 1e9
    # dominant kernel: on the single-launch path the whole layer is one kernel, so its
    # average duration is the timed region (events on the replay stream) / launches
    kernel = "fused_t1_kernel" if fused else "moe_layer_unfused"
    avg_launch_us = us_per_layer / launches_per_layer if fused else us_per_layer
    kgbps = abytes / (avg_launch_us * 1e-6) / 1e9
    roofline = {
        "bound": "hbm",
        "kernel": kernel,
        "achieved": round(kgbps, 1),
        "peak": HBM_PEAK_GBPS,
        "unit": "GB/s",
        "frac": round(kgbps / HBM_PEAK_GBPS, 4),
        "traffic": read_traffic(kernel),
        "bytes_per_launch": abytes,
        "avg_launch_us": round(avg_launch_us, 3),
        "timing": "events on the replay stream around the K timed graph replays, divided "
                  "by the kernel launches they contain (steps x layers)",
        "eager_call_us_median": round(eager_us, 3),
    }
    rec = {
        "metric": METRIC,
        "value": round(us_per_layer, 3),
        "unit": "us/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "config": {"workload": "q30_moe_layer_t1", "T": T, "E": E, "H": H, "I": I, "k": k,
                   "format": "fp4_e2m1", "group": G, "layers_per_step": args.layers,
                   "active_bytes_per_layer": abytes, "path": args.path},
        "achieved_GBps": round(gbps, 1),
        "roofline": roofline,
        "device": torch.cuda.get_device_name(dev),
        "kernel_source_hash": kernel_source_hash(),
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline()
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
