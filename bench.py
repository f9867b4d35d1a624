"""Benchmark: microseconds per packed-MoE layer at T=1 on the 30B-A3B expert shape
(E=128, H=2048, I=768, top-8, FP4 E2M1, group 32), with achieved HBM GB/s over the bytes
of the active experts' packed weights and scales, against the 8 TB/s MI355X peak.

One step = one token through a stack of 48 distinct layer weight sets (about 1 GB of
active expert bytes per step, four times the 256 MB last-level cache), each layer =
routing from fp32 logits + gate_up + SiLU*up + down + top-k combine in one
`moe_fp4_layer` call.  The layers are captured once into a graph; the timed region
replays it K times between events on the capturing stream.  Inputs (weights, scales,
activations, logits) are synthetic and already resident in device memory.

`--workload` selects the other sizes (Q30 at T = 4, 16, 64; the 48-layer chained
512-expert stack at T = 1, 8; a tiny INT4 layer; the dense INT4 GEMV with N = 256, 8192,
34816 at T = 1, 4 and N = 34816 at T = 2), each timed the same way.

Prints one JSON line.  `--gpus` above 1 exits: this benchmark is single-GPU.
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
FP4, INT4, FP8 = 1, 0, 2

# Synthetic workloads (sizes of the 30B-A3B and 512-expert MoE layers, a tiny INT4 layer and
# the dense INT4 GEMV).  `layers` distinct weight sets are rotated so that one timed pass
# reads well past the 256 MB last-level cache; `chain` feeds each layer's output to the
# next as both input and residual.
WORKLOADS = {
    "q30_moe_layer_t1": dict(kind="moe", T=1, E=128, H=2048, I=768, k=8, group=32, fmt=FP4,
                             scales=(0.002, 0.01), logits="normal", layers=48),
    "q30_moe_layer_t4": dict(kind="moe", T=4, E=128, H=2048, I=768, k=8, group=32, fmt=FP4,
                             scales=(0.002, 0.01), logits="normal+bias", layers=48),
    "q30_moe_layer_t8": dict(kind="moe", T=8, E=128, H=2048, I=768, k=8, group=32, fmt=FP4,
                             scales=(0.002, 0.01), logits="normal+bias", layers=32),
    "q30_moe_layer_t16": dict(kind="moe", T=16, E=128, H=2048, I=768, k=8, group=32, fmt=FP4,
                              scales=(0.002, 0.01), logits="normal+bias", layers=24),
    "q30_moe_layer_t32": dict(kind="moe", T=32, E=128, H=2048, I=768, k=8, group=32, fmt=FP4,
                              scales=(0.002, 0.01), logits="normal+bias", layers=16),
    "q30_moe_layer_t64": dict(kind="moe", T=64, E=128, H=2048, I=768, k=8, group=32, fmt=FP4,
                              scales=(0.002, 0.01), logits="normal+bias", layers=12),
    "w512_stack_t1": dict(kind="moe", T=1, E=512, H=2048, I=512, k=10, group=32, fmt=FP4,
                          scales=(0.002, 0.01), logits="zipf", layers=48, chain=True),
    "w512_stack_t8": dict(kind="moe", T=8, E=512, H=2048, I=512, k=10, group=32, fmt=FP4,
                          scales=(0.002, 0.01), logits="zipf", layers=48, chain=True),
    "q30_router_layer_t1": dict(kind="moe", T=1, E=128, H=2048, I=768, k=8, group=32, fmt=FP4,
                                scales=(0.002, 0.01), logits="router", layers=48),
    "q30_router_layer_t4": dict(kind="moe", T=4, E=128, H=2048, I=768, k=8, group=32, fmt=FP4,
                                scales=(0.002, 0.01), logits="router", layers=48),
    "q30_fp8_layer_t1": dict(kind="moe", T=1, E=128, H=2048, I=768, k=8, group=32, fmt=FP8,
                             scales=(0.002, 0.01), logits="normal", layers=48),
    "q30_fp8_layer_t4": dict(kind="moe", T=4, E=128, H=2048, I=768, k=8, group=32, fmt=FP8,
                             scales=(0.002, 0.01), logits="normal+bias", layers=24),
    "q30_fp8_layer_t16": dict(kind="moe", T=16, E=128, H=2048, I=768, k=8, group=32, fmt=FP8,
                              scales=(0.002, 0.01), logits="normal+bias", layers=12),
    "q30_fp8_layer_t64": dict(kind="moe", T=64, E=128, H=2048, I=768, k=8, group=32, fmt=FP8,
                              scales=(0.002, 0.01), logits="normal+bias", layers=8),
    "q30_mixed_layer_t1": dict(kind="moe", T=1, E=128, H=2048, I=768, k=8, group=32, fmt=FP4,
                               scales=(0.002, 0.01), logits="normal", layers=48, int2_frac=0.25),
    "q30_codebook_layer_t1": dict(kind="moe", T=1, E=128, H=2048, I=768, k=8, group=32,
                                  fmt=FP4, scales=(0.002, 0.01), logits="normal", layers=48,
                                  int2_frac=0.25, fexc_frac=0.25),
    "q30_codebook_layer_t16": dict(kind="moe", T=16, E=128, H=2048, I=768, k=8, group=32,
                                   fmt=FP4, scales=(0.002, 0.01), logits="normal+bias",
                                   layers=24, int2_frac=0.25, fexc_frac=0.25),
    "tiny_moe_layer_t1": dict(kind="moe", T=1, E=8, H=256, I=128, k=2, group=32, fmt=INT4,
                              scales=(0.005, 0.02), logits="normal", layers=48),
    "gemv_int4_n256_t1": dict(kind="gemv", T=1, K=5120, N=256, group=128, copies=48),
    "gemv_int4_n8192_t1": dict(kind="gemv", T=1, K=5120, N=8192, group=128, copies=48),
    "gemv_int4_n8192_t4": dict(kind="gemv", T=4, K=5120, N=8192, group=128, copies=48),
    "gemv_int4_n34816_t1": dict(kind="gemv", T=1, K=5120, N=34816, group=128, copies=8),
    "gemv_int4_n34816_t2": dict(kind="gemv", T=2, K=5120, N=34816, group=128, copies=8),
    "gemv_int4_n34816_t4": dict(kind="gemv", T=4, K=5120, N=34816, group=128, copies=8),
    # the same GEMVs on the prepacked (tile-contiguous) weights
    "gemv_int4_tiled_n256_t1": dict(kind="gemv", T=1, K=5120, N=256, group=128, copies=48,
                                    tiled=True),
    "gemv_int4_tiled_n8192_t1": dict(kind="gemv", T=1, K=5120, N=8192, group=128, copies=48,
                                     tiled=True),
    "gemv_int4_tiled_n8192_t4": dict(kind="gemv", T=4, K=5120, N=8192, group=128, copies=48,
                                     tiled=True),
    "gemv_int4_tiled_n34816_t1": dict(kind="gemv", T=1, K=5120, N=34816, group=128, copies=8,
                                      tiled=True),
    "gemv_int4_tiled_n34816_t2": dict(kind="gemv", T=2, K=5120, N=34816, group=128, copies=8,
                                      tiled=True),
    "gemv_int4_tiled_n34816_t4": dict(kind="gemv", T=4, K=5120, N=34816, group=128, copies=8,
                                      tiled=True),
}
DEFAULT_WORKLOAD = "q30_moe_layer_t1"
KERNEL_SOURCES = {
    "fused_layer_kernel": ("dqg_fused.hip", "dqg_device.hpp", "dqg_internal.hpp"),
    "gemv_ex_kernel": ("dqg_experts.hip", "dqg_device.hpp", "dqg_internal.hpp"),
    "gemv_tok_kernel": ("dqg_experts.hip", "dqg_device.hpp", "dqg_internal.hpp"),
    "moe_layer_multi_launch": ("dqg_kernels.hip", "dqg_experts.hip", "dqg_device.hpp",
                               "dqg_internal.hpp"),
}


def expert_bytes(H, I, G, kb=2):
    """Packed bytes + bf16 scales of one expert (gate_up and down); kb = K indices per byte
    (2 for the 4-bit formats, 1 for FP8)."""
    return (H // kb) * (2 * I) + (H // G) * (2 * I) * 2 + (I // kb) * H + (I // G) * H * 2


def active_bytes(H, I, G, k):
    per_expert = expert_bytes(H, I, G)
    return k * per_expert, per_expert


def kernel_source_hash(kernel=None) -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "dequant_gemv_amd", "csrc")
    files = KERNEL_SOURCES.get(kernel) if kernel else None
    for f in sorted(files or os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def _bf16_scales(shape, lo, hi, g, device):
    import torch
    return (torch.rand(shape, device=device, generator=g) * (hi - lo) + lo).to(torch.bfloat16)


def _logits(w, g, device):
    """Router logits of one layer: N(0,1), plus a per-expert N(0, 0.5) bias
    ("normal+bias"), or -1.1 ln(1 + perm(e)) + N(0,1) over a per-layer permutation
    ("zipf")."""
    import torch
    T, E = w["T"], w["E"]
    lg = torch.randn((T, E), device=device, generator=g, dtype=torch.float32)
    if w["logits"] == "normal+bias":
        lg += 0.5 * torch.randn((E,), device=device, generator=g)[None, :]
    elif w["logits"] == "zipf":
        perm = torch.randperm(E, device=device, generator=g).to(torch.float32)
        lg += -1.1 * torch.log1p(perm)[None, :]
    return lg


def _codes(w, shape, g, device):
    """Packed weight bytes: uniform over 0..255 (4-bit formats: every nibble uniform), or
    for FP8 the E4M3 codes of N(0, 2) values (torch's float8_e4m3fn cast)."""
    import torch
    if w["fmt"] == FP8:
        v = 2.0 * torch.randn(shape, device=device, generator=g)
        return v.to(torch.float8_e4m3fn).view(torch.uint8)
    return torch.randint(0, 256, shape, dtype=torch.uint8, device=device, generator=g)


def _expert_formats(w, g, device):
    """Mixed layers: per-layer seeded random int2_frac and fexc_frac shares of the experts are
    INT2 and FE-XC (their codes are the first quarter of the slab's random bytes, every byte a
    valid INT2 or FE-XC code)."""
    import torch
    f2, fx = w.get("int2_frac", 0.0), w.get("fexc_frac", 0.0)
    if f2 <= 0 and fx <= 0:
        return None
    E = w["E"]
    f = torch.full((E,), FP4, dtype=torch.uint8, device=device)
    cold = torch.randperm(E, device=device, generator=g)
    n2, nx = int(round(f2 * E)), int(round(fx * E))
    f[cold[:n2]] = 3           # INT2
    f[cold[n2:n2 + nx]] = 4    # FE-XC
    return f


def build_moe_workload(w, seed: int = 0, device="cuda"):
    """Layer weight sets drawn on the device: packed bytes uniform over 0..255 (every
    nibble uniform), scales uniform in the workload's range rounded to bf16, x ~ N(0,1)
    in bf16, logits as in _logits, one set per layer.  Router workloads ("router") draw a
    router weight W_r ~ N(0, 1/sqrt(H)) in bf16 [H, E] per layer instead of logits."""
    import torch
    T, E, H, I, G = w["T"], w["E"], w["H"], w["I"], w["group"]
    kb = 1 if w["fmt"] == FP8 else 2
    lo, hi = w["scales"]
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = []
    for _ in range(w["layers"]):
        out.append(dict(
            w_gu=_codes(w, (E, H // kb, 2 * I), g, device),
            s_gu=_bf16_scales((E, H // G, 2 * I), lo, hi, g, device),
            w_d=_codes(w, (E, I // kb, H), g, device),
            s_d=_bf16_scales((E, I // G, H), lo, hi, g, device),
            logits=None if w["logits"] == "router" else _logits(w, g, device),
            wr=(torch.randn((H, E), device=device, generator=g) / H ** 0.5).to(torch.bfloat16)
            if w["logits"] == "router" else None,
            efmt=_expert_formats(w, g, device),
            cb=(2.0 * torch.randn((E, 2, 2, 256, 8), device=device, generator=g)).to(torch.bfloat16)
            if w.get("fexc_frac", 0.0) > 0 else None,
        ))
    x = torch.randn((T, H), device=device, generator=g).to(torch.bfloat16)
    return x, out


def build_gemv_workload(w, seed: int = 0, device="cuda"):
    """`copies` weight sets W ~ N(0, 0.02) [K, N], symmetric INT4 per group of 128 along K
    (s = bf16(absmax / 7), q = clamp(rint(w / s), -8, 7), nibble q + 8, low nibble = even
    K), and x ~ N(0,1) bf16 [T, K]."""
    import torch
    T, K, N, G = w["T"], w["K"], w["N"], w["group"]
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    sets = []
    for _ in range(w["copies"]):
        wf = torch.randn((K, N), device=device, generator=g) * 0.02
        wg = wf.view(K // G, G, N)
        s = (wg.abs().amax(dim=1) / 7.0).to(torch.bfloat16)
        s = torch.where(s == 0, torch.ones_like(s), s)
        q = torch.clamp(torch.round(wg / s.float()[:, None, :]), -8, 7).to(torch.int16) + 8
        q = q.view(K, N).to(torch.uint8)
        packed = (q[0::2] | (q[1::2] << 4)).contiguous()
        sets.append(dict(w=packed, s=s.contiguous()))
        del wf, wg, q
    x = torch.randn((T, K), device=device, generator=g).to(torch.bfloat16)
    return x, sets


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def host_layer(L, k):
    """Host copy of one timed layer's logits and of its routed experts' slabs only (dicts
    keyed by expert id: the oracle looks experts up by id)."""
    import numpy as np
    import torch
    from oracle import moe_oracle as O
    lg = L["logits"].cpu().numpy()
    ids, _ = O.topk_route(lg, k)
    sl = {}
    for name in ("w_gu", "s_gu", "w_d", "s_d"):
        t = L[name] if L[name].dtype == torch.uint8 else L[name].view(torch.int16)
        sl[name] = {int(e): t[int(e)].cpu().numpy() for e in np.unique(ids)}
        if L[name].dtype != torch.uint8:
            sl[name] = {e: a.view(np.uint16) for e, a in sl[name].items()}
    return lg, sl


def oracle_layer_out(x_bits, lg, sl, k, group, fmt, residual_bits=None):
    from oracle import moe_oracle as O
    out, _, _ = O.moe_layer(x_bits, lg, k, sl["w_gu"], sl["s_gu"], sl["w_d"], sl["s_d"], group,
                            fmt, residual_bits=residual_bits)
    return out


def within_method_tolerance(gpu_bits, want):
    """|gpu - oracle| <= 1e-2 rms(oracle) + 1 bf16 ulp of the oracle value, per element."""
    import numpy as np
    g = (gpu_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    rms = float(np.sqrt(np.mean(np.square(want))))
    a = np.abs(want)
    ulp = np.where(a > 0, 2.0 ** (np.maximum(np.floor(np.log2(np.where(a > 0, a, 1.0))), -126) - 7),
                   2.0 ** -133)
    err = np.abs(g - want)
    return bool(np.all(err <= 1e-2 * rms + ulp)), float(np.max(err / (1e-2 * rms + ulp)))


def cpu_baseline(timed, x_bits, k, group, fmt, budget_s: float = 10.0):
    """The float64 oracle on layers the GPU timed (their routed experts copied to the
    host), after checking the GPU's outputs of those layers against it.  Two legs: one
    thread with one BLAS thread (median µs per layer), then one worker thread per core of
    this process's CPU set (at most 16), each running whole layers with one BLAS thread
    (µs per layer = wall time / layers).  numpy releases the GIL inside its array loops, so
    the threads run side by side; threads rather than processes keep every CPU worker
    inside this one process.  `timed` lists (logits, slabs, gpu_out_bits) per layer."""
    import concurrent.futures as cf
    import statistics
    from threadpoolctl import threadpool_limits
    worst = 0.0
    for lg, sl, gpu_bits in timed[:4]:  # parity first
        ok, ratio = within_method_tolerance(gpu_bits, oracle_layer_out(x_bits, lg, sl, k, group,
                                                                          fmt))
        if not ok:
            raise SystemExit(f"cpu_baseline: GPU output of a timed layer is outside the "
                             f"tolerance (worst ratio {ratio:.3f})")
        worst = max(worst, ratio)
    times, t_one = [], 0.0
    with threadpool_limits(limits=1):
        while t_one < budget_s / 2 and len(times) < 4 * len(timed):
            lg, sl, _ = timed[len(times) % len(timed)]
            t0 = time.perf_counter()
            oracle_layer_out(x_bits, lg, sl, k, group, fmt)
            dt = time.perf_counter() - t0
            times.append(dt)
            t_one += dt
    one_us = statistics.median(times) * 1e6
    ncpu = min(len(os.sched_getaffinity(0)), 16)
    # all cores: as many layers as one core did in its leg, times the core count, so that
    # the leg also takes about budget_s / 2 at perfect scaling

    def one_layer(i):
        lg, sl, _ = timed[i % len(timed)]
        oracle_layer_out(x_bits, lg, sl, k, group, fmt)

    n_all = max(ncpu, int(len(times) * ncpu))
    with threadpool_limits(limits=1), cf.ThreadPoolExecutor(max_workers=ncpu) as ex:
        list(ex.map(one_layer, range(ncpu)))            # threads started
        t0 = time.perf_counter()
        list(ex.map(one_layer, range(n_all)))
        t_all = time.perf_counter() - t0
    return {"value": round(t_all / n_all * 1e6, 1), "unit": "us/layer", "cores": ncpu,
            "kind": "oracle",
            "sample": f"{n_all} GPU-timed layers (route + routed experts + combine, float64 "
                      f"numpy) on {ncpu} worker threads, {t_all:.1f} s wall; "
                      f"value = wall time / layers",
            "single_thread": {"value": round(one_us, 1), "unit": "us/layer", "cores": 1,
                              "sample": f"median of {len(times)} layers, {t_one:.1f} s"},
            "cpu_model": cpu_model(),
            "parity_checked": f"GPU outputs of {min(4, len(timed))} timed layers within the "
                              f"tolerance (worst ratio {worst:.3f}) before timing"}


def read_traffic(kernel: str, workload: str):
    """HBM traffic per launch from the committed rocprofv3 counter summary, or None when
    the kernel's sources changed since the counters were taken."""
    p = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
    except Exception:
        return None
    e = d.get(f"{kernel}/{workload}")
    if not e or e.get("source_hash") != kernel_source_hash(kernel):
        return None
    return e.get("hbm_bytes_per_launch")


class GraphTimer:
    """fn() captured once into a graph on `stream` (after one eager warm-up call on that
    stream); timed replays with events recorded on `stream`."""

    def __init__(self, fn, stream):
        import torch
        # every input was written on the default stream: finish that work first, or the
        # caching allocator's reuse of freed temporaries can overlap buffers used here
        torch.cuda.synchronize()
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            fn()
        stream.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph, stream=stream):
            fn()
        self.stream = stream

    def replay(self, n):
        import torch
        with torch.cuda.stream(self.stream):
            for _ in range(n):
                self.graph.replay()

    def timed(self, steps, warmup):
        """warmup untimed replays, then `steps` replays between two events; ms per replay."""
        import torch
        self.replay(warmup)
        self.stream.synchronize()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(self.stream)
        self.replay(steps)
        e1.record(self.stream)
        e1.synchronize()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    def rounds(self, n_rounds=3, samples=30):
        """n_rounds rounds of `samples` replays, each between its own pair of events:
        per round the median and the min-max (ms per replay)."""
        import statistics
        import torch
        out = []
        for _ in range(n_rounds):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(samples + 1)]
            with torch.cuda.stream(self.stream):
                ev[0].record(self.stream)
                for i in range(samples):
                    self.graph.replay()
                    ev[i + 1].record(self.stream)
            ev[-1].synchronize()
            t = [ev[i].elapsed_time(ev[i + 1]) for i in range(samples)]
            out.append({"median": statistics.median(t), "min": min(t), "max": max(t)})
        return out


def time_graph(fn, stream, steps, warmup):
    """ms per replay of fn() captured into a graph (see GraphTimer)."""
    return GraphTimer(fn, stream).timed(steps, warmup)


def calibration(dev, stream, B):
    """Context recorded with every run: the achievable read bandwidth (one streaming read of
    a 2 GiB buffer per replay, 10 replays), a 1 GiB device copy (read + write GB/s) and the
    per-launch floor of a graph of 256 one-element kernels."""
    import torch
    rb = 2 << 30
    rbuf = torch.empty(rb, dtype=torch.uint8, device=dev).fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    gt = GraphTimer(lambda: B.stream_read(rbuf, sink), stream)
    ms_read = gt.timed(10, 3)
    read_rounds = gt.rounds(3, 10)
    del gt, rbuf
    torch.cuda.empty_cache()
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    ms = time_graph(lambda: dst.copy_(src), stream, 10, 3)
    t = torch.zeros(1, device=dev)

    def tiny():
        for _ in range(256):
            t.add_(1.0)
    ms_tiny = time_graph(tiny, stream, 10, 3)
    del src, dst
    torch.cuda.empty_cache()
    return {"achievable_read_GBps": round(rb / (ms_read * 1e-3) / 1e9, 1),
            "read_rounds_GBps": [round(rb / (r["median"] * 1e-3) / 1e9, 1) for r in read_rounds],
            "read_bytes": rb,
            "copy_GBps": round(2 * n / (ms * 1e-3) / 1e9, 1),
            "graph_launch_floor_us": round(ms_tiny * 1000.0 / 256, 3)}


def distinct_experts(logits, k):
    """Distinct experts the router selects for a [T, E] logits tensor (accounting only)."""
    import torch
    return int(torch.unique(torch.topk(logits, k, dim=1).indices).numel())


def bench_moe(w, args, dev, stream, B):
    import numpy as np
    import torch
    T, E, H, I, k, G = (w[s] for s in ("T", "E", "H", "I", "k", "group"))
    fmt = {FP4: B.FMT_FP4_E2M1, INT4: B.FMT_INT4, FP8: B.FMT_FP8_E4M3}[w["fmt"]]
    flags = {"auto": 0, "unfused": B.PATH_NO_FUSED, "gemv": B.PATH_FORCE_GEMV | B.PATH_NO_FUSED,
             "mfma": B.PATH_FORCE_MFMA | B.PATH_NO_FUSED}[args.path]
    x, layers = build_moe_workload(w, device=dev)
    ws = B.moe_workspace(T, H, I, E, k, dev)
    chain = w.get("chain", False)
    router = w["logits"] == "router"
    xs = [x] + [torch.empty_like(x) for _ in layers]
    lbuf = torch.empty((T, E), dtype=torch.float32, device=dev)
    rws = B.router_logits_workspace(T, H, E, dev) if router else None
    torch.cuda.synchronize()

    def call(l, L, out=None, workspace=None):
        xin = xs[l] if chain else x
        out = xs[l + 1] if out is None else out
        workspace = ws if workspace is None else workspace
        if router:
            B.moe_fp4_layer_from_hidden(xin, L["wr"], k, L["w_gu"], L["s_gu"], L["w_d"],
                                        L["s_d"], G, fmt, residual=xin if chain else None,
                                        out=out, workspace=workspace, flags=flags)
            return
        if L["efmt"] is not None:
            B.moe_fp4_layer_mixed(xin, L["logits"], k, L["w_gu"], L["s_gu"], L["w_d"], L["s_d"],
                                  L["efmt"], G, codebooks=L["cb"], residual=xin if chain else None,
                                  out=out, workspace=workspace, flags=flags)
            return
        B.moe_fp4_layer(xin, L["logits"], k, L["w_gu"], L["s_gu"], L["w_d"], L["s_d"], G, fmt,
                        residual=xin if chain else None, out=out, workspace=workspace,
                        flags=flags)

    def one_pass():
        for l, L in enumerate(layers):
            call(l, L)

    gt = GraphTimer(one_pass, stream)
    ms_per_step = gt.timed(args.steps, args.warmup)
    n_layers = len(layers)
    us_per_layer = ms_per_step * 1000.0 / n_layers
    rounds = gt.rounds(3, 30)

    # validation of the timed run: no error bit in the workspace; the last replay's output
    # of layer l0 equals an eager call's bit for bit; and it meets the method's tolerance
    # against the oracle on that layer's host copy (the eager call reads the same inputs)
    err_word = int(ws[:4].view(torch.int32).item())
    if err_word != 0:
        raise SystemExit(f"bench: workspace error word {err_word:#x} after the timed replays")
    l0 = n_layers // 2
    ws_v = B.moe_workspace(T, H, I, E, k, dev)
    eager = torch.empty_like(x)
    with torch.cuda.stream(stream):
        call(l0, layers[l0], out=eager, workspace=ws_v)
    stream.synchronize()
    replay_bits = xs[l0 + 1].view(torch.int16).cpu().numpy().view(np.uint16)
    if not np.array_equal(replay_bits, eager.view(torch.int16).cpu().numpy().view(np.uint16)):
        raise SystemExit("bench: a replayed layer's output differs from an eager call")
    validation = {"error_word": 0, "replay_equals_eager_layer": l0}
    plain = not router and layers[0]["efmt"] is None
    timed_host = []
    if plain:
        xin_bits = (xs[l0] if chain else x).view(torch.int16).cpu().numpy().view(np.uint16)
        lg, sl = host_layer(layers[l0], k)
        ok, ratio = within_method_tolerance(
            replay_bits, oracle_layer_out(xin_bits, lg, sl, k, G, w["fmt"],
                                          residual_bits=xin_bits if chain else None))
        if not ok:
            raise SystemExit(f"bench: timed layer {l0} is outside the tolerance ({ratio:.3f})")
        validation["oracle_worst_ratio_layer"] = round(ratio, 4)
        if not chain and args.workload == DEFAULT_WORKLOAD and not args.no_cpu_baseline:
            x_bits = x.view(torch.int16).cpu().numpy().view(np.uint16)
            for l in range(min(n_layers, 12)):
                lg, sl = host_layer(layers[l], k)
                timed_host.append((lg, sl, xs[l + 1].view(torch.int16).cpu().numpy()
                                   .view(np.uint16)))
            validation["cpu_x"] = x_bits
    del ws_v

    # warm figure (context, not HBM): one layer's weights called n_layers times in a graph
    warm_us = None
    if not chain and not args.graph_only:
        def warm_pass():
            for l in range(n_layers):
                call(0, layers[0])
        warm_us = GraphTimer(warm_pass, stream).timed(max(5, args.steps // 4), 3) * 1000.0 / n_layers

    # context only: events right before and after each eager layer call (includes the
    # host launch overhead that the graph replay hides)
    eager_us = None
    if not args.graph_only:
        per = []
        with torch.cuda.stream(stream):
            for rep in range(3):
                for l, L in enumerate(layers):
                    a0 = torch.cuda.Event(enable_timing=True)
                    a1 = torch.cuda.Event(enable_timing=True)
                    a0.record(stream)
                    call(l, L)
                    a1.record(stream)
                    per.append((a0, a1))
        stream.synchronize()
        eager_us = sorted(a0.elapsed_time(a1) * 1000.0 for a0, a1 in per)[len(per) // 2]
    separate_us = None
    if router and not args.graph_only:
        # context: the same layers as two calls, the router call then the logits-taking layer
        def two_calls():
            for l, L in enumerate(layers):
                B.router_logits(x, L["wr"], logits=lbuf, workspace=rws)
                B.moe_fp4_layer(x, lbuf, k, L["w_gu"], L["s_gu"], L["w_d"], L["s_d"], G, fmt,
                                out=xs[l + 1], workspace=ws, flags=flags)
        separate_us = time_graph(two_calls, stream, args.steps, args.warmup) * 1000.0 / n_layers

    per_expert = expert_bytes(H, I, G, 1 if w["fmt"] == FP8 else 2)
    lgs = [L["logits"] if not router else x.float() @ L["wr"].float() for L in layers]
    n_active = [distinct_experts(lg, k) for lg in lgs]
    abytes = sum(n_active) * per_expert / n_layers  # mean active bytes per layer
    n_int2 = 0.0
    if layers[0]["efmt"] is not None:  # mixed: INT2 experts stream half the packed bytes
        i2 = expert_bytes(H, I, G, 4)
        tot = 0
        for lg, L in zip(lgs, layers):
            act = torch.unique(torch.topk(lg, k, dim=1).indices)
            n2 = int((L["efmt"][act] >= 3).sum())   # INT2 and FE-XC: 2 bits per weight
            n_int2 += n2
            tot += (act.numel() - n2) * per_expert + n2 * i2
            if L["cb"] is not None:                   # codebooks of the routed FE-XC experts
                tot += int((L["efmt"][act] == 4).sum()) * 2 * 2 * 256 * 8 * 2
        abytes = tot / n_layers
        n_int2 /= n_layers
    if router:
        abytes += H * E * 2                         # the router weight
    # the single-launch layer takes T <= 8 (for T > 1 a token's down rows must fill whole
    # 256-row chunks), E <= 512, H % 256 == 0, H <= 2048, I % 128 == 0
    fused = (args.path == "auto" and T <= 8 and E <= 512 and H % 256 == 0 and H <= 2048
             and I % 128 == 0 and (T == 1 or (k * (I // (1 if w["fmt"] == FP8 else 2))) % 256 == 0))
    gbps = abytes / (us_per_layer * 1e-6) / 1e9
    # the single-launch path runs the whole layer in one kernel, so its average duration
    # is the timed region (events on the replay stream) / launches; the multi-launch path
    # is reported per layer (schedule + gate_up + down)
    kernel = "fused_layer_kernel" if fused else "moe_layer_multi_launch"
    roofline = {
        "bound": "hbm",
        "kernel": kernel,
        "achieved": round(gbps, 1),
        "peak": HBM_PEAK_GBPS,
        "unit": "GB/s",
        "frac": round(gbps / HBM_PEAK_GBPS, 4),
        "traffic": read_traffic(kernel, args.workload),
        "bytes_per_launch": round(abytes),
        "avg_launch_us": round(us_per_layer, 3),
        "timing": "events on the replay stream around the K timed graph replays, divided "
                  "by the layer calls they contain (steps x layers)",
        "rounds_us_per_layer": [{key: round(r[key] * 1000.0 / n_layers, 3) for key in r}
                                for r in rounds],
    }
    if eager_us is not None:
        roofline["eager_call_us_median"] = round(eager_us, 3)
    if warm_us is not None:
        roofline["warm_us_per_layer"] = round(warm_us, 3)
    if router:
        roofline["router_in_launch"] = fused and E <= 128 and E % 8 == 0 and T <= 4
        if separate_us is not None:
            roofline["router_call_then_layer_us"] = round(separate_us, 3)
    config = {"workload": args.workload, "T": T, "E": E, "H": H, "I": I, "k": k,
              "format": {FP4: "fp4_e2m1", INT4: "int4", FP8: "fp8_e4m3"}[w["fmt"]], "group": G,
              "layers_per_step": n_layers, "chained": chain, "path": args.path,
              "active_experts_per_layer_mean": round(sum(n_active) / n_layers, 2),
              "active_bytes_per_layer": round(abytes)}
    if layers[0]["efmt"] is not None:
        config["int2_experts_share"] = w.get("int2_frac", 0.0)
        config["fexc_experts_share"] = w.get("fexc_frac", 0.0)
        config["two_bit_active_experts_per_layer_mean"] = round(n_int2, 2)
    cpu = None
    if timed_host:
        cpu = cpu_baseline(timed_host, validation.pop("cpu_x"), k, G, w["fmt"])
    validation.pop("cpu_x", None)
    return dict(value=round(us_per_layer, 3), unit="us/layer", ms_per_step=ms_per_step,
                achieved_GBps=round(gbps, 1), roofline=roofline, config=config,
                validation=validation, cpu_baseline=cpu)


def bench_gemv(w, args, dev, stream, B):
    import numpy as np
    import torch
    T, K, N, G = w["T"], w["K"], w["N"], w["group"]
    tiled = bool(w.get("tiled"))
    x, sets = build_gemv_workload(w, device=dev)
    if tiled:  # prepacked once, outside the timed region (weights prepared before inference)
        for S_ in sets:
            S_["wt"], S_["st"] = B.packed_gemv_int4_prepack(S_["w"], S_["s"], G)
        for S_ in sets[1:]:
            del S_["w"], S_["s"]
        def call(S_, y, ws_):
            B.packed_gemv_int4_tiled(x, S_["wt"], S_["st"], N, G, y=y, workspace=ws_)
    else:
        def call(S_, y, ws_):
            B.packed_gemv_int4(x, S_["w"], S_["s"], G, y=y, workspace=ws_)
    mkws = lambda: B.gemv_workspace(T, K, N, G, dev)
    ws = mkws()
    ys = [torch.empty((T, N), dtype=torch.bfloat16, device=dev) for _ in sets]
    torch.cuda.synchronize()

    def one_pass():
        for S_, y in zip(sets, ys):
            call(S_, y, ws)

    gt = GraphTimer(one_pass, stream)
    ms_per_step = gt.timed(args.steps, args.warmup)
    rounds = gt.rounds(3, 30)
    us = ms_per_step * 1000.0 / len(sets)
    # validation: error word clear, a replayed call equals an eager one, and the oracle bound
    # on 512 sampled columns of that call
    if ws is not None and int(ws[:4].view(torch.int32).item()) != 0:
        raise SystemExit("bench: GEMV workspace error word set after the timed replays")
    y_e = torch.empty_like(ys[0])
    with torch.cuda.stream(stream):
        call(sets[0], y_e, mkws())
    stream.synchronize()
    rb = ys[0].view(torch.int16).cpu().numpy().view(np.uint16)
    if not np.array_equal(rb, y_e.view(torch.int16).cpu().numpy().view(np.uint16)):
        raise SystemExit("bench: a replayed GEMV differs from an eager call")
    from oracle import moe_oracle as O
    cols = np.unique(np.random.default_rng(0).choice(N, min(N, 512), replace=False))
    want = O.packed_gemv(x.view(torch.int16).cpu().numpy().view(np.uint16),
                         sets[0]["w"].cpu().numpy(),
                         sets[0]["s"].view(torch.int16).cpu().numpy().view(np.uint16), G,
                         cols=cols)
    ok, ratio = within_method_tolerance(rb[:, cols], want)
    if not ok:
        raise SystemExit(f"bench: timed GEMV outside the tolerance ({ratio:.3f})")
    abytes = (K // 2) * N + (K // G) * N * 2
    gbps = abytes / (us * 1e-6) / 1e9
    # (up to 4 tokens: gemv_tok_kernel, its matrix-core body from 2 tokens, either layout)
    kernel = "gemv_tok_kernel" if T <= 4 else "gemv_ex_kernel"
    roofline = {"bound": "hbm", "kernel": kernel, "achieved": round(gbps, 1),
                "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
                "traffic": read_traffic(kernel, args.workload), "bytes_per_launch": abytes,
                "avg_launch_us": round(us, 3),
                "timing": "events around the K timed graph replays / GEMV calls (one "
                          "launch per call)",
                "rounds_us_per_call": [{key: round(r[key] * 1000.0 / len(sets), 3) for key in r}
                                       for r in rounds]}
    config = {"workload": args.workload, "T": T, "K": K, "N": N, "group": G, "format": "int4",
              "weight_copies": len(sets), "layout": "prepacked" if tiled else "[K/2, N]"}
    return dict(value=round(us, 3), unit="us/call", ms_per_step=ms_per_step,
                achieved_GBps=round(gbps, 1), roofline=roofline, config=config,
                validation={"error_word": 0, "replay_equals_eager": True,
                            "oracle_worst_ratio_512_cols": round(ratio, 4)},
                cpu_baseline=None)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-calibration", action="store_true")
    ap.add_argument("--graph-only", action="store_true",
                    help="skip the context measurements that are not graph replays of the timed "
                         "layers (eager per-call timing, the cache-warm figure): profiling runs")
    ap.add_argument("--path", choices=["auto", "unfused", "gemv", "mfma"], default="auto",
                    help="MoE kernel path: auto, or force the multi-launch path with its "
                         "automatic / vector-ALU-only / matrix-core-only expert tiles")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES bytes (3 times); "
                         "used to scale rocprofv3 FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: every kernel "
              "of this library runs on a single GPU", file=sys.stderr)
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
    w = WORKLOADS[args.workload]
    stream = torch.cuda.Stream(device=dev)
    stream.wait_stream(torch.cuda.current_stream(dev))
    cal = None if args.no_calibration else calibration(dev, stream, B)
    r = (bench_moe if w["kind"] == "moe" else bench_gemv)(w, args, dev, stream, B)
    roof = r["roofline"]
    if cal:
        roof["achievable_read_GBps"] = cal["achievable_read_GBps"]
        roof["frac_of_achievable"] = round(roof["achieved"] / cal["achievable_read_GBps"], 4)
    rec = {
        "metric": METRIC if args.workload == DEFAULT_WORKLOAD else
        f"{r['unit'].replace('us/', 'µs per ')} and achieved HBM GB/s vs peak ({args.workload})",
        "value": r["value"],
        "unit": r["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic (seeded device RNG; inputs resident in HBM)",
        "config": r["config"],
        "achieved_GBps": r["achieved_GBps"],
        "roofline": roof,
        "calibration": cal,
        "validation": r["validation"],
        "device": torch.cuda.get_device_name(dev),
        "kernel_source_hash": kernel_source_hash(),
    }
    if r.get("cpu_baseline"):
        rec["cpu_baseline"] = r["cpu_baseline"]
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
