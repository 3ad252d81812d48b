#!/usr/bin/env python3
"""LatentMoE layer forward throughput on one MI355X.

One step = one moe_forward over a batch of T tokens: down-projection, fp32
router, top-K/softmax, expert histogram/scan/scatter, the two grouped expert
GEMMs, combine and up-projection, all in libmoe.so on HBM-resident inputs.

    python bench.py [--config 5] [--steps 20] [--warmup 5] [--gpus 1]
    python bench.py --paired      # standard vs latent at the ablation shapes
    python bench.py --paired router_at_d   # router on the latent vs on x at d
    python bench.py --config 5 --hipblaslt  # torch's bf16 GEMM on the layer's shapes

Prints one JSON line.  `value` is tokens/s of the whole layer.  `roofline`
describes the dominant kernel (the grouped expert GEMMs): its algorithmic
FLOPs or bytes per launch over its average launch duration, measured with HIP
events on the launch stream during the timed region (the library's stage
timer).  `cpu_baseline` is the plain fp64 CPU oracle timed on a bounded sample
of the same workload (rank 0, N = 1 only).
"""
import argparse
import json
import os
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "LatentMoE layer tokens/sec on 1 MI355X; % MFMA peak (prefill), % HBM BW (decode)"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA
PEAK_F32_TFLOPS = 157.3        # MI355X fp32 (matrix)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
CPU_SAMPLE = {1: 64, 2: 1536, 3: 3072, 4: 64, 5: 384, 11: 3072, 12: 64, 13: 384}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def expert_weight_bytes_per_matrix(cfg):
    el = cfg.latent * cfg.ffn
    if cfg.expert == "nvfp4":
        return el / 2 + el / 16 + 4
    if cfg.expert == "fp8":
        return el + 4
    return el * (4 if cfg.expert == "f32" else 2)


def expert_kernel(cfg):
    """The kernel the library runs the grouped expert GEMMs on: the skinny
    kernel for batches of up to 128 tokens when l and m are multiples of 256,
    the tiled MFMA kernel otherwise (fp32 kernel for an all-fp32 layer); with
    NVFP4 weights on 256-row tiles (64 or more rows per expert on average) the
    remainder tiles run as a second launch, gemm_fp4_rem_kernel."""
    if cfg.act == "f32":
        return "gemm_f32_kernel"
    if cfg.T <= 128 and cfg.latent % 256 == 0 and cfg.ffn % 256 == 0:
        return "skinny_kernel"
    if cfg.expert == "nvfp4" and cfg.T * cfg.top_k >= 64 * cfg.n_experts:
        return "gemm_bf16_kernel + gemm_fp4_rem_kernel"
    return "gemm_bf16_kernel"


def layer_bytes(cfg, touched):
    """Algorithmic HBM bytes of one layer step: both weight matrices of every
    touched expert, the projection, router and shared-expert weights, x and y.
    Intermediates (latent rows, expert-sorted rows, logits) are not counted."""
    act = 4 if cfg.act == "f32" else 2
    b = 2 * touched * expert_weight_bytes_per_matrix(cfg)
    if cfg.has_latent_proj:
        b += 2 * cfg.d * cfg.latent * act
    b += cfg.n_experts * (cfg.d if cfg.router_on_x else cfg.latent) * 4 + cfg.n_experts * 4
    b += 2 * cfg.n_shared * cfg.shared_ffn * cfg.d * (1 if cfg.shared_fp8 else act)
    b += 2 * cfg.T * cfg.d * act
    return b


TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic_counters.json")


def source_sha256():
    """Hash of the kernel sources (csrc/*), which the counter summary is tied to."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for src in sorted(glob.glob(os.path.join(ROOT, "sparse_moe_layer_fwd_amd", "csrc", "*"))):
        with open(src, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload):
    """HBM bytes per launch of the grouped expert GEMM from the committed counter
    summary (FETCH_SIZE, WRITE_SIZE scaled by a plain-copy calibration), or None
    when the kernel sources changed since the counters were taken."""
    if not os.path.exists(TRAFFIC_JSON):
        return None
    with open(TRAFFIC_JSON) as f:
        rec = json.load(f)
    w = rec.get("workloads", {}).get(workload)
    if source_sha256() != rec.get("source_sha256") or not w:
        return None
    if w.get("fetch_kib_per_dispatch") is None or w.get("write_kib_per_dispatch") is None:
        return None
    return (w["fetch_kib_per_dispatch"] * rec["fetch_scale"] +
            w["write_kib_per_dispatch"] * rec["write_scale"]) * 1024.0


def is_grouped_expert_kernel(name):
    """The grouped expert GEMMs: the tiled kernel with a remainder list (its
    third template argument, the remainder tile height, is nonzero; the dense
    projections have 0), the NVFP4 remainder-tile kernel, or the skinny expert
    kernel."""
    import re
    m = re.search(r"gemm_bf16_kernel<\s*\d+,\s*\d+,\s*(\d+),", name)
    return bool(m and int(m.group(1)) > 0) or "skinny_kernel<" in name or "gemm_fp4_rem_kernel<" in name


def traffic_summary(indir, config_ids):
    """Summarise rocprofv3 --pmc runs into profiles/traffic_counters.json:
    indir/fetch<N> and indir/write<N> hold the FETCH_SIZE and WRITE_SIZE runs
    of `bench.py --config N`, indir/copy_fetch and indir/copy_write those of
    `bench.py --copy-calibration 1024`.  Per workload, the counters of the
    grouped expert GEMM dispatches are averaged (KiB per dispatch); the copy
    gives the factor from each counter to HBM bytes.  Prints a markdown table."""
    import csv
    import glob
    from sparse_moe_layer_fwd_amd.workloads import CONFIGS

    def dispatches(sub, counter):
        per = {}
        for path in glob.glob(os.path.join(indir, sub, "**", "*counter_collection.csv"), recursive=True):
            with open(path) as f:
                for row in csv.DictReader(f):
                    if row["Counter_Name"] != counter:
                        continue
                    key = (path, row["Dispatch_Id"])
                    rec = per.setdefault(key, [row["Kernel_Name"], 0.0])
                    rec[1] += float(row["Counter_Value"])
        return list(per.values())

    copy_kib = 1024.0 * 1024.0                  # the 1 GiB copy, in KiB
    fetch_copy = max(v for _, v in dispatches("copy_fetch", "FETCH_SIZE"))
    write_copy = max(v for _, v in dispatches("copy_write", "WRITE_SIZE"))
    out = {"source_sha256": source_sha256(), "fetch_scale": round(copy_kib / fetch_copy, 4),
           "write_scale": round(copy_kib / write_copy, 4), "workloads": {}}
    rows = ["| workload | GEMM calls | FETCH_SIZE KiB | WRITE_SIZE KiB | read GB | write GB | traffic GB / GEMM |",
            "|---|---|---|---|---|---|---|"]
    for cid in config_ids:
        cfg = CONFIGS[cid]
        f = [(k, v) for k, v in dispatches("fetch%d" % cid, "FETCH_SIZE") if is_grouped_expert_kernel(k)]
        w = [(k, v) for k, v in dispatches("write%d" % cid, "WRITE_SIZE") if is_grouped_expert_kernel(k)]
        if not f or not w:
            continue
        # per grouped GEMM: every matched dispatch summed, over the GEMM calls
        # (an NVFP4 GEMM is two launches, its remainder tiles the second)
        nf = len([k for k, _ in f if "gemm_fp4_rem_kernel<" not in k])
        nw = len([k for k, _ in w if "gemm_fp4_rem_kernel<" not in k])
        fk, wk = sum(v for _, v in f) / max(1, nf), sum(v for _, v in w) / max(1, nw)
        out["workloads"][cfg.name] = {"kernel": " | ".join(sorted({k for k, _ in f})), "dispatches": nf,
                                      "fetch_kib_per_dispatch": round(fk), "write_kib_per_dispatch": round(wk)}
        rd, wr = fk * out["fetch_scale"] * 1024 / 1e9, wk * out["write_scale"] * 1024 / 1e9
        rows.append("| %s | %d | %d | %d | %.3f | %.3f | %.3f |" % (cfg.name, nf, fk, wk, rd, wr, rd + wr))
    with open(TRAFFIC_JSON, "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    print("calibration: FETCH_SIZE %.0f KiB, WRITE_SIZE %.0f KiB per 1 GiB copy" % (fetch_copy, write_copy))
    print("\n".join(rows))


def cpu_baseline(cfg, seed, sample):
    """Time the fp64 oracle on the first `sample` tokens of the same workload."""
    import numpy as np  # noqa: F401
    import oracle
    from sparse_moe_layer_fwd_amd.workloads import Workload
    sub = cfg.replace(T=sample)
    wl = Workload(sub, seed)
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()
                     if i.get("user_api") == "blas"] or [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    oracle.forward(wl, sub)
    dt = time.perf_counter() - t0
    return {"value": sample / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": "first %d of the %d tokens of the same workload (seed %d), whole layer in "
                      "fp64 numpy incl. per-expert weight decode; %.2f s" % (sample, cfg.T, seed, dt)}


class GpuTelemetry:
    """Samples the GPU's graphics clock (MHz) and socket power (W) through
    amdsmi every `period` seconds on a host thread while steps run.  Any
    failure (no amdsmi, no permission) leaves the record empty."""

    def __init__(self, period=0.02):
        self.period, self.clk, self.pwr = period, [], []
        self._stop = threading.Event()
        self._t = None
        self.error = None

    def _loop(self, smi, h):
        while not self._stop.is_set():
            try:
                c = smi.amdsmi_get_clock_info(h, smi.AmdSmiClkType.GFX)
                self.clk.append(float(c["clk"]))
                pw = smi.amdsmi_get_power_info(h)
                v = pw.get("current_socket_power", "N/A")
                if v in ("N/A", None):
                    v = pw.get("average_socket_power", "N/A")
                if v not in ("N/A", None):
                    self.pwr.append(float(v))
            except Exception as e:      # keep timing, report why the record is empty
                self.error = repr(e)
                return
            time.sleep(self.period)

    def start(self):
        try:
            import amdsmi as smi
            smi.amdsmi_init()
            h = smi.amdsmi_get_processor_handles()[0]
        except Exception as e:
            self.error = repr(e)
            return self
        self._t = threading.Thread(target=self._loop, args=(smi, h), daemon=True)
        self._t.start()
        return self

    def stop(self):
        self._stop.set()
        if self._t is not None:
            self._t.join()
        return self

    def record(self):
        r = {"samples": len(self.clk), "period_s": self.period}
        # instantaneous readings: samples that fall between kernels read idle
        # clocks, so the median is the figure under load
        med = lambda v: sorted(v)[len(v) // 2]
        if self.clk:
            r.update({"sclk_mhz_median": med(self.clk), "sclk_mhz_mean": round(sum(self.clk) / len(self.clk), 1),
                      "sclk_mhz_min": min(self.clk), "sclk_mhz_max": max(self.clk)})
        if self.pwr:
            r.update({"power_w_median": med(self.pwr), "power_w_mean": round(sum(self.pwr) / len(self.pwr), 1),
                      "power_w_max": max(self.pwr)})
        if self.error:
            r["error"] = self.error
        return r


def hipblaslt_context(cfg, steps, warmup):
    """torch.nn.functional.linear in bf16 (hipBLASLt on ROCm) on the layer's
    dense shapes: the two latent projections and one dense GEMM with the FLOPs
    of a grouped expert launch (T*K rows, l -> m).  Random bf16 operands, fp32
    accumulation; context for the library's own kernels, not part of the layer."""
    import torch
    import torch.nn.functional as F

    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(0)
    shapes = {}
    if cfg.latent != cfg.d:
        shapes["down_proj"] = (cfg.T, cfg.latent, cfg.d)     # rows, out, in
        shapes["up_proj"] = (cfg.T, cfg.d, cfg.latent)
    shapes["expert_up_as_dense"] = (cfg.T * cfg.top_k, cfg.ffn, cfg.latent)
    out = {"what": "torch bf16 linear (hipBLASLt) on %s shapes" % cfg.name, "steps": steps}
    for name, (m, n, k) in shapes.items():
        a = torch.randn((m, k), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
        w = (torch.randn((n, k), generator=g, device=dev, dtype=torch.float32) / k ** 0.5).to(torch.bfloat16)
        for _ in range(warmup):
            F.linear(a, w)
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(steps):
            F.linear(a, w)
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / steps
        tf = 2.0 * m * n * k / (ms * 1e-3) / 1e12
        out[name] = {"m_n_k": [m, n, k], "ms": round(ms, 4), "tflops": round(tf, 1),
                     "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
        del a, w
        torch.cuda.empty_cache()
    return out


def forced_workload(cfg, seed):
    """The layer's workload with every token routed to the same K experts
    (experts 0, N/K, 2N/K, ...: a large router bias on them): every expert GEMM
    then runs full-height row tiles only, a dense-like ablation of the same
    layer and FLOPs."""
    import numpy as np
    from sparse_moe_layer_fwd_amd.workloads import Workload

    class Forced(Workload):
        def b_router(self):
            b = np.zeros(cfg.n_experts, np.float32)
            b[np.arange(cfg.top_k) * (cfg.n_experts // cfg.top_k)] = 50.0
            return b
    return Forced(cfg, seed)


def time_layer(cfg, cfg_id, seed, steps, warmup, telemetry_ms=500.0, forced=False, phases=True):
    """Build the layer with seeded weights, warm up, then time `steps`
    back-to-back moe_forward calls on the current stream (inputs resident in
    HBM) with the library's per-stage timer on."""
    import torch
    from sparse_moe_layer_fwd_amd import binding as B
    from sparse_moe_layer_fwd_amd.layer import DeviceLayer, x_to_device
    from sparse_moe_layer_fwd_amd.workloads import Workload

    dev = torch.device("cuda:0")
    log("bench: config %d %s, generating weights" % (cfg_id, cfg.name))
    t0 = time.perf_counter()
    wl = forced_workload(cfg, seed) if forced else Workload(cfg, seed)
    layer = DeviceLayer.from_workload(wl, device=dev, threads=16)
    x = x_to_device(wl, dev)
    y = torch.empty((cfg.T, cfg.d), dtype=layer.act_torch_dtype(), device=dev)
    ws = layer.new_workspace(cfg.T)
    torch.cuda.synchronize()
    log("bench: inputs resident in HBM (%.1f s); warmup %d" % (time.perf_counter() - t0, warmup))

    for _ in range(warmup):
        layer.forward(x, ws=ws, y=y)
    y2, idx, gate, counts = layer.forward(x, ws=ws, y=y, routing=True)
    torch.cuda.synchronize()
    counts_np = counts.cpu().numpy()

    stream = torch.cuda.current_stream(dev)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # one more event per step boundary: per-step times for the median
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    B.moe_profile_read()                      # clear
    B.moe_profile_enable(True)
    torch.cuda.synchronize()
    start.record(stream)
    marks[0].record(stream)
    for i in range(steps):
        layer.forward(x, ws=ws, y=y)
        marks[i + 1].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    B.moe_profile_enable(False)
    stages = B.moe_profile_read()
    ms_step = start.elapsed_time(end) / steps
    per_step = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(steps))
    step_stats = {"median": round(per_step[len(per_step) // 2], 5), "min": round(per_step[0], 5),
                  "max": round(per_step[-1], 5)}
    log("bench: %.3f ms/step (median %.3f)" % (ms_step, step_stats["median"]))
    # the grouped expert GEMMs' two phases (full row tiles, remainder tiles),
    # timed as separate launches over further steps after the timed region
    split_ms = None
    if phases:
        B.moe_profile_enable(2)
        for _ in range(steps):
            layer.forward(x, ws=ws, y=y)
        torch.cuda.synchronize()
        B.moe_profile_enable(False)
        split = B.moe_profile_read()
        if split["expert_up_rem"][0]:
            split_ms = {"steps": steps}
            split_ms.update({k: round(split[k][1] / steps, 5) for k in
                             ("expert_up", "expert_up_rem", "expert_down", "expert_down_rem")})
    # clock and power under the same load: sampled over further steps (at
    # least telemetry_ms) after the timed region, which stays untouched
    telemetry = None
    if telemetry_ms > 0:
        n_tel = max(steps, int(telemetry_ms / max(ms_step, 1e-3)) + 1)
        tel = GpuTelemetry(period=0.01).start()
        for _ in range(n_tel):
            layer.forward(x, ws=ws, y=y)
        torch.cuda.synchronize()
        tel.stop()
        telemetry = dict(tel.record(), steps=n_tel)
    del layer, ws, x, y
    torch.cuda.empty_cache()
    return {"ms_step": ms_step, "stages": stages, "counts": counts_np,
            "touched": int((counts_np > 0).sum()), "telemetry": telemetry, "step_stats": step_stats,
            "phases": split_ms}


# Paired comparisons: (metric, (role a, role b), [(regime, config of a, config of b)])
PAIRS = {
    # standard MoE (128 experts top-6 at d) against LatentMoE (512 experts
    # top-22 at l = d/4) at equal d and m
    "ablation": ("standard vs latent MoE layer at the ablation shapes (paired, 1 MI355X)",
                 ("standard", "latent"), [("prefill", 6, 3), ("decode", 7, 8)]),
    # the latent layer with its router on the latent and no shared experts,
    # against the same layer with the router and two shared experts at d
    "router_at_d": ("LatentMoE with router on the latent vs router and shared experts at d "
                    "(paired, 1 MI355X)", ("latent", "router_at_d"), [("prefill", 3, 9), ("decode", 8, 10)]),
    # the latent layers with bf16 experts against the same layers with FP8
    # (E4M3) expert weights and activations
    "fp8": ("LatentMoE with bf16 vs FP8 experts (paired, 1 MI355X)", ("bf16", "fp8"),
            [("prefill", 3, 11), ("decode", 4, 12)]),
}


def paired(args):
    """Time the two layers of each pair back to back, in prefill and in batch
    decode.  One JSON line: per layer the step time, tokens/s, FLOP per token,
    algorithmic bytes per token and the expert weight bytes a step reads, and
    the ratios of the second layer to the first."""
    from sparse_moe_layer_fwd_amd.workloads import CONFIGS
    metric, (ra, rb), pairs = PAIRS[args.paired]
    out = {"metric": metric, "unit": "ms per step", "steps": args.steps, "warmup": args.warmup,
           "data": "synthetic (seeded random weights and inputs)", "pairs": []}
    for regime, a_id, b_id in pairs:
        rec = {"regime": regime}
        for role, cid in ((ra, a_id), (rb, b_id)):
            cfg = CONFIGS[cid]
            r = time_layer(cfg, cid, args.seed, args.steps, args.warmup, phases=False)
            rec[role] = {
                "workload": cfg.name, "T": cfg.T, "d": cfg.d, "latent": cfg.latent,
                "n_experts": cfg.n_experts, "top_k": cfg.top_k, "ffn": cfg.ffn,
                "ms_per_step": round(r["ms_step"], 5),
                "tokens_per_s": round(cfg.T / (r["ms_step"] * 1e-3), 1),
                "flop_per_token": cfg.flops() / cfg.T,
                "bytes_per_token": layer_bytes(cfg, r["touched"]) / cfg.T,
                "expert_weight_gb_per_step": round(2 * r["touched"] * expert_weight_bytes_per_matrix(cfg) / 1e9, 4),
                "experts_touched": r["touched"],
                "stages_ms_per_step": {k: round(v[1] / max(1, args.steps), 5) for k, v in r["stages"].items() if v[0]},
            }
        s_, l_ = rec[ra], rec[rb]
        rec["%s_over_%s" % (rb, ra)] = {
            "time": round(l_["ms_per_step"] / s_["ms_per_step"], 4),
            "flop_per_token": round(l_["flop_per_token"] / s_["flop_per_token"], 4),
            "bytes_per_token": round(l_["bytes_per_token"] / s_["bytes_per_token"], 4),
            "expert_weight_bytes_per_step": round(l_["expert_weight_gb_per_step"] / s_["expert_weight_gb_per_step"], 4),
        }
        out["pairs"].append(rec)
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=5,
                    help="layer configuration 1-13 (default 5: the Ultra-like NVFP4 prefill layer, "
                         "the largest configuration on one GPU)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-sample", type=int, default=None, help="tokens for the CPU oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--telemetry-ms", type=float, default=500.0,
                    help="sample clock and power over this many ms of extra steps after the timed "
                         "region (0: off, e.g. under a profiler)")
    ap.add_argument("--paired", nargs="?", const="ablation", choices=sorted(PAIRS), default=None,
                    help="time a pair of layers instead: 'ablation' (standard vs latent, "
                         "configurations 6/3 and 7/8), 'router_at_d' (3/9 and 8/10) or 'fp8' "
                         "(bf16 vs FP8 experts, 3/11 and 4/12)")
    ap.add_argument("--expert-dtype", choices=["bf16", "nvfp4", "fp8"], default=None,
                    help="ablation: the chosen layer with its routed experts in another storage type")
    ap.add_argument("--forced-routing", action="store_true",
                    help="ablation: every token routed to the same K experts (full row tiles only)")
    ap.add_argument("--hipblaslt", action="store_true",
                    help="context only: time torch's bf16 GEMM (hipBLASLt) on the layer's dense shapes")
    ap.add_argument("--no-phases", action="store_true",
                    help="skip the phase-split steps after the timed region (for profiler runs)")
    ap.add_argument("--traffic-summary", metavar="DIR", default=None,
                    help="write profiles/traffic_counters.json from rocprofv3 FETCH_SIZE / WRITE_SIZE runs "
                         "under DIR (fetch<N>, write<N>, copy_fetch, copy_write); no GPU needed")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (scales HBM traffic counters)")
    args = ap.parse_args()
    if args.traffic_summary:
        traffic_summary(args.traffic_summary, [2, 3, 4, 5, 11, 12, 13])
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: it measures the layer on a single MI355X "
              "(--gpus %d requested). Multi-GPU expert parallelism is not implemented." % args.gpus,
              file=sys.stderr, flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calibration:
        # A plain copy of known size: under rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE
        # it gives the factor between the counters and real HBM bytes.
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        for _ in range(max(1, args.steps)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_launch": n, "launches": max(1, args.steps)}))
        return

    from sparse_moe_layer_fwd_amd.workloads import CONFIGS

    if args.hipblaslt:
        print(json.dumps(hipblaslt_context(CONFIGS[args.config], args.steps, args.warmup)), flush=True)
        return
    if args.paired:
        paired(args)
        return

    cfg = CONFIGS[args.config]
    if args.expert_dtype and args.expert_dtype != cfg.expert:
        cfg = cfg.replace(name=cfg.name + "+%s_experts" % args.expert_dtype, expert=args.expert_dtype)
    if args.forced_routing:
        cfg = cfg.replace(name=cfg.name + "+forced_routing")
    r = time_layer(cfg, args.config, args.seed, args.steps, args.warmup, args.telemetry_ms,
                   forced=args.forced_routing, phases=not args.no_phases)
    ms_step, stages, counts_np, touched = r["ms_step"], r["stages"], r["counts"], r["touched"]

    # dominant kernel: the grouped expert GEMMs (two launches per step)
    n_up, ms_up = stages["expert_up"]
    n_dn, ms_dn = stages["expert_down"]
    launches = n_up + n_dn
    avg_ms = (ms_up + ms_dn) / max(1, launches)
    # algorithmic work of one grouped launch: 2*T*K*l*m FLOP, and the weights of
    # every touched expert (one matrix) read once; expert-sorted rows are
    # intermediates of this implementation and are not counted
    flops_launch = 2.0 * cfg.T * cfg.top_k * cfg.latent * cfg.ffn
    bytes_launch = touched * expert_weight_bytes_per_matrix(cfg)
    # the MFMA peak of the contraction's own dtype (NVFP4 weights are decoded
    # to bf16 and run on the bf16 MFMA)
    peak_f = {"f32": PEAK_F32_TFLOPS, "fp8": PEAK_FP8_TFLOPS}.get(cfg.expert, PEAK_BF16_TFLOPS)
    t_mfma = flops_launch / (peak_f * 1e12)
    t_hbm = bytes_launch / (PEAK_HBM_GBS * 1e9)
    if t_hbm > t_mfma:
        ach = bytes_launch / (avg_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": None}
    else:
        ach = flops_launch / (avg_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": peak_f, "unit": "TFLOP/s",
                "frac": round(ach / peak_f, 4), "traffic": None}
    roof["traffic"] = measured_traffic(cfg.name)
    roof.update({"kernel": "grouped expert GEMM (%s)" % expert_kernel(cfg),
                 "launches": launches, "avg_launch_ms": round(avg_ms, 5),
                 "algorithmic_flops_per_launch": flops_launch,
                 "algorithmic_bytes_per_launch": bytes_launch})

    result = {
        "metric": METRIC,
        "value": round(cfg.T / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        # per-step HIP-event times over the same timed steps
        "ms_per_step_stats": r["step_stats"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"nvfp4": "nvfp4-weights/bf16", "fp8": "fp8-e4m3"}.get(cfg.expert, cfg.act),
        "data": "synthetic (seeded random weights and inputs, shapes of the layer configuration)",
        "config": {"workload": cfg.name, "T": cfg.T, "d": cfg.d, "latent": cfg.latent,
                   "n_experts": cfg.n_experts, "top_k": cfg.top_k, "ffn": cfg.ffn,
                   "n_shared": cfg.n_shared, "expert_dtype": cfg.expert,
                   "shared_fp8": cfg.shared_fp8, "router_on_x": cfg.router_on_x,
                   "zipf_s": cfg.zipf_s, "experts_touched": touched,
                   "max_rows_per_expert": int(counts_np.max()), "parallelism": "single GPU"},
        "layer_tflops": round(cfg.flops() / (ms_step * 1e-3) / 1e12, 2),
        # whole-layer HBM fraction (algorithmic bytes / step time / 8 TB/s), the
        # decode-regime figure
        "layer_hbm_frac": round(layer_bytes(cfg, touched) / (ms_step * 1e-3) / (PEAK_HBM_GBS * 1e9), 4),
        "stages_ms_per_step": {k: round(v[1] / max(1, args.steps), 5) for k, v in stages.items() if v[0]},
        # the grouped GEMMs split into their full-tile and remainder-tile
        # launches (ms per step; further steps after the timed region)
        "grouped_gemm_phases_ms_per_step": r["phases"],
        # graphics clock and socket power, sampled over further steps of the
        # same workload right after the timed region
        "gpu_telemetry": r["telemetry"],
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        sample = args.cpu_sample or CPU_SAMPLE.get(args.config, 64)
        log("bench: CPU oracle baseline on %d tokens" % sample)
        result["cpu_baseline"] = cpu_baseline(cfg, args.seed, sample)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
