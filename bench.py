#!/usr/bin/env python3
"""Throughput of the single-GPU MoE expert layer on MI355X.

One step = route -> permute -> grouped fc1+SwiGLU -> grouped fc2 [-> shared experts]
-> combine over one batch of seeded synthetic tokens, all inputs resident in HBM.
Between timed steps (outside the HIP-event brackets of each step) a 512 MiB buffer is
written so the 256 MB Infinity Cache holds nothing of the previous step.

By default every bf16 layer workload runs one after the other (dense 8-expert, the
fine-grained 64-expert layer with shared experts, the skewed 32-expert layer, the
expert-tensor-parallel shard); the dense layer is the headline. Prints one JSON line:
the headline's MoE-layer tokens/s, its grouped GEMM's TFLOP/s and fraction of the bf16
MFMA peak, permute and combine GB/s and fraction of HBM bandwidth, per-stage median /
p10 / p90 / CV, the roofline of the dominant kernel (grouped fc1) measured with HIP
events on the stream the kernels run on, its backward and FP8-payload steps, the CPU
oracle timed on a bounded sample, and under "configs" the same figures for every
workload.

    python bench.py [--steps K] [--warmup W] [--workload all|NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA (AMD spec)
PEAK_F32_TFLOPS = 157.3       # MI355X fp32 vector
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E
METRIC = "MoE-layer tokens/sec; grouped-GEMM TFLOP/s (% bf16 MFMA peak); permute GB/s"
HEADLINE = "dense8_bf16"
SUITE = ["dense8_bf16", "fine64_shared2_bf16", "skew32_zipf_bf16", "etp_shard32_bf16",
         "decode8_bf16", "decode64_shared2_bf16"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_GEMM_SOURCES = ["grouped_gemm.hip", "lds_dma.hpp", "common.hpp", "decode_gemm.hip"]


def gemm_source_sha16() -> str:
    """sha256 (first 16 hex digits) of the grouped GEMM kernels' sources."""
    h = hashlib.sha256()
    for n in _GEMM_SOURCES:
        with open(os.path.join(_HERE, "routing_permute_grouped_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# HBM-side traffic of the dominant kernels per launch (per step for the masked decode
# GEMM): rocprofv3 FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0 bytes, the factors measured on a
# device copy of known size (bench.py --copy-calibration 256), each taken at the GEMM
# sources whose hash is stored beside it. A workload without an entry, or an entry taken
# at other sources, reports null: the counters describe the kernel they were read on.
# kind: fc1 (forward), wgrad_fc1 (backward), fp8_fc1 (FP8 payload), masked (decode).
TRAFFIC = {
    "fc1": {
        "dense8_bf16": (4316417075, "ec23b0769012bcba"),
        "etp_shard32_bf16": (1034965483, "ec23b0769012bcba"),
        "fine64_shared2_bf16": (2384506166, "ec23b0769012bcba"),
        "skew32_zipf_bf16": (5397533361, "ec23b0769012bcba"),
    },
    "wgrad_fc1": {
        "dense8_bf16": (8144705579, "ec23b0769012bcba"),
    },
    "fp8_fc1": {
        "dense8_bf16": (2480918277, "ec23b0769012bcba"),
    },
    "masked": {
        "decode8_bf16": (2920594913, "ec23b0769012bcba"),
        "decode64_shared2_bf16": (1167546070, "ec23b0769012bcba"),
    },
}


def fc1_kernel_name(E: int, m_cap: int) -> str:
    """The kernel the library runs the bf16 fc1 on: the LDS ring while the experts have at
    most about five 256-row blocks each (at most 64 experts), else the two-stage kernel."""
    return "gg_ring_kernel<kFc1>" if E <= 64 and m_cap <= 5 * 256 * E else "gg_bf16_kernel<kFc1>"


class HipEvent:
    """A timing-only HIP event recorded on a given stream. It is created with
    hipEventDisableSystemFence: a default event's record makes a system-scope fence (an L2
    writeback and invalidate), which costs microseconds at every stage boundary and starts
    the next stage with a cold L2; a timing event needs none of it (the record still waits
    for the work before it on the stream). Same interface as torch.cuda.Event."""
    _lib = None

    def __init__(self):
        import ctypes
        if HipEvent._lib is None:
            lib = ctypes.CDLL("libamdhip64.so")
            lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
            lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
            HipEvent._lib = lib
        self._ct = ctypes
        self.h = ctypes.c_void_p()
        rc = HipEvent._lib.hipEventCreateWithFlags(ctypes.byref(self.h), 0x20000000)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def record(self, stream) -> None:
        rc = HipEvent._lib.hipEventRecord(self.h, self._ct.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_time(self, end: "HipEvent") -> float:
        """Milliseconds from this event to ``end`` (both recorded and completed)."""
        ms = self._ct.c_float()
        rc = HipEvent._lib.hipEventElapsedTime(self._ct.byref(ms), self.h, end.h)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        if HipEvent._lib is not None and self.h:
            HipEvent._lib.hipEventDestroy(self.h)


def traffic(kind: str, workload: str):
    """(bytes, note) for the kernel ``kind`` on ``workload``: the stored counter reading
    when it was taken at the current GEMM sources, else (None, why)."""
    ent = TRAFFIC.get(kind, {}).get(workload)
    if ent is None:
        return None, "no counter reading for this workload"
    val, sha = ent
    if sha != gemm_source_sha16():
        return None, f"counters taken at GEMM sources {sha}; current {gemm_source_sha16()}"
    return val, f"rocprofv3 FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0 at GEMM sources {sha}"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="all",
                    help="all (the four bf16 layer workloads, dense8_bf16 first and the "
                         "headline, then the two decode workloads on the masked layout) or "
                         "one workload name")
    ap.add_argument("--cpu-sample-tokens", type=int, default=4096)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the headline's step with the FP8 (e4m3, MX-scaled) payload "
                         "(reported under \"fp8_payload\")")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the headline's timed backward pass (reported under "
                         "\"backward\")")
    ap.add_argument("--no-split-k", action="store_true",
                    help="give the grouped GEMMs no workspace (every tile whole)")
    ap.add_argument("--shared-overlap", choices=["auto", "none", "start", "after-route"],
                    default="auto",
                    help="run the shared experts' GEMM on a second stream (with its own "
                         "split-K workspace), from the step's start or after the router; the "
                         "per-stage times of route / permute then include waiting for CUs. "
                         "auto: from the start for decode steps (masked layout), where the "
                         "shared GEMM leaves most CUs idle, none for the others")
    ap.add_argument("--graph", action="store_true",
                    help="also capture one contiguous-layout step (without a second stream) in "
                         "a HIP graph and time K replays of it (reported under `graph`)")
    ap.add_argument("--flush-mib", type=int, default=512,
                    help="MiB written between timed steps to evict the Infinity Cache (0: none)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only copy MIB MiB device-to-device 10 times (a kernel of known "
                         "traffic for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE), then 10 "
                         "more timed with events (the device-copy rate), then exit")
    return ap.parse_args()


def copy_calibration(mib: int) -> None:
    import torch
    n = mib * 1024 * 1024 // 2
    a = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(10):
        b.copy_(a)
    torch.cuda.synchronize()
    # ten more, timed: the rate a plain device copy reaches (read + write bytes), the
    # ceiling the permute and combine are compared with
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / 10
    nbytes = mib * 1024 * 1024
    print(json.dumps({"copy_calibration_MiB": mib, "launches": 20,
                      "bytes_read_per_launch": nbytes, "bytes_written_per_launch": nbytes,
                      "us_per_copy_timed": us, "GBps_read_plus_write": 2 * nbytes / us / 1e3}))


def cpu_baseline(inp: dict, cfg, tokens: int, min_seconds: float = 10.0) -> dict:
    """The oracle as it stands, on the first ``tokens`` tokens of the same workload,
    repeated (at most 8 passes) until about ``min_seconds`` of CPU work is timed. Each
    pass calls the oracle's stage functions in the order of ``oracle.forward`` and times
    each stage with time.perf_counter."""
    from threadpoolctl import threadpool_info

    from oracle import moe_oracle as orc
    x = inp["x"][:tokens]
    E = inp["w1"].shape[0]
    stages = {"route": 0.0, "layout": 0.0, "permute": 0.0, "experts": 0.0, "shared": 0.0,
              "combine": 0.0}
    passes = 0
    while passes == 0 or (sum(stages.values()) < min_seconds and passes < 8):
        t = time.perf_counter()
        if "topk_idx" in inp:
            idx, w = inp["topk_idx"][:tokens], inp["topk_w"][:tokens].astype(np.float64)
        else:
            idx, w, _ = orc.route(x, inp["wg"], cfg.k, cfg.dtype, inp.get("bias"), False)
        t1 = time.perf_counter()
        lay = orc.dispatch_layout(idx, E, cfg.m_tile)
        t2 = time.perf_counter()
        xp = orc.permute(x, lay)
        t3 = time.perf_counter()
        _, y = orc.grouped_swiglu(xp, lay["offsets"], inp["w1"], inp["w3"], inp["w2"], cfg.dtype)
        t4 = time.perf_counter()
        sh = None
        if "ws1" in inp:
            sh = orc.shared_experts(x, inp["ws1"], inp["ws3"], inp["ws2"], cfg.dtype)
        t5 = time.perf_counter()
        orc.combine(y, lay["dst_row"], w, cfg.dtype, sh)
        t6 = time.perf_counter()
        for name, dt in zip(stages, (t1 - t, t2 - t1, t3 - t2, t4 - t3, t5 - t4, t6 - t5)):
            stages[name] += dt
        passes += 1
    total = sum(stages.values())
    pools = threadpool_info()
    threads = max([p.get("num_threads", 1) for p in pools] + [1])
    blas = sorted({f"{p.get('internal_api')} {p.get('version')}" for p in pools
                   if p.get("user_api") == "blas"})
    return {"value": passes * tokens / total, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "affinity_cores": len(os.sched_getaffinity(0)), "blas": blas,
            "stage_s_per_pass": {n: v / passes for n, v in stages.items()},
            "sample": f"first {tokens} tokens of {cfg.name} with every expert's weights; "
                      f"{passes} oracle pass(es) (routing, layout, permute, float64 "
                      f"experts, combine) took {total:.2f} s"}


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)

    import torch

    import workloads as W

    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    names = SUITE if args.workload == "all" else [args.workload]
    overlap_arg = args.shared_overlap
    results, head_inp = {}, None
    for i, name in enumerate(names):
        t0 = time.perf_counter()
        inp = W.generate(W.preset(name), seed=0)
        cfg = inp["cfg"]
        print(f"[bench] {name}: inputs drawn in {time.perf_counter() - t0:.1f} s",
              file=sys.stderr, flush=True)

        def up(a):
            a = np.ascontiguousarray(a)
            if a.dtype == np.uint16:
                return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
            return torch.from_numpy(a).to(dev)

        d = {n: up(a) for n, a in inp.items() if isinstance(a, np.ndarray)}
        args.shared_overlap = overlap_arg
        if args.shared_overlap == "auto":
            args.shared_overlap = "start" if cfg.cap else "none"
        if cfg.cap:
            rec = bench_masked(args, cfg, d, inp)
        else:
            rec = run_contiguous(args, cfg, d, headline=(i == 0))
        results[name] = rec
        print(f"[bench] {name}: {rec['value'] / 1e6:.3f} M tokens/s", file=sys.stderr, flush=True)
        if i == 0:
            head_inp = inp
        del d, inp
        torch.cuda.empty_cache()
    rec = results[names[0]]
    if len(names) > 1:
        rec["configs"] = {n: config_summary(r) for n, r in results.items()}
    if not args.no_cpu_baseline and not W.preset(names[0]).cap:
        cfg0 = head_inp["cfg"]
        rec["cpu_baseline"] = cpu_baseline(head_inp, cfg0, min(args.cpu_sample_tokens, cfg0.T))
    print(json.dumps(rec), flush=True)


def config_summary(r: dict) -> dict:
    """The per-workload figures carried under "configs" in the JSON line."""
    keys = ["value", "unit", "ms_per_step", "config", "roofline", "grouped_gemm_tflops",
            "grouped_gemm_frac_bf16_peak", "fc1_tflops", "fc2_tflops", "fc1_frac_bf16_peak",
            "fc2_frac_bf16_peak", "permute_GBps", "permute_frac_hbm", "combine_GBps",
            "combine_frac_hbm", "route_us", "stage_us_mean", "stage_us_spread",
            "expert_rows_min_max", "assignments", "padded"]
    return {k: r[k] for k in keys if k in r}


def run_contiguous(args, cfg, d: dict, headline: bool) -> dict:
    """Time the layer on the contiguous (padded-segment) layout; the headline workload
    also times its backward and its FP8-payload step unless switched off."""
    import torch

    import routing_permute_grouped_amd as rpg

    T, D, F, E, k, mt = cfg.T, cfg.D, cfg.F, cfg.E, cfg.k, cfg.m_tile
    dev = d["x"].device
    tdt = d["x"].dtype
    m_cap = rpg.moe_capacity(T, k, E, mt)
    i32 = dict(dtype=torch.int32, device=dev)
    buf = {
        "idx": d.get("topk_idx", torch.empty((T, k), **i32)),
        "w": d.get("topk_w", torch.empty((T, k), dtype=torch.float32, device=dev)),
        "x_perm": torch.empty((m_cap, D), dtype=tdt, device=dev),
        "counts": torch.empty(E, **i32), "offsets": torch.empty(E + 1, **i32),
        "dst_row": torch.empty((T, k), **i32), "src_row": torch.empty(m_cap, **i32),
        "tile_expert": torch.empty(m_cap // mt, **i32), "dev_err": torch.empty(1, **i32),
        "workspace": torch.empty(max(4, rpg.moe_permute_workspace_bytes(T, k, E)),
                                 dtype=torch.uint8, device=dev),
        "h": torch.empty((m_cap, F), dtype=tdt, device=dev),
        "y": torch.empty((m_cap, D), dtype=tdt, device=dev),
        "out": torch.empty((T, D), dtype=tdt, device=dev),
    }
    gws = None if args.no_split_k else rpg.grouped_workspace(dev)
    shared = None
    if cfg.n_shared:
        shared = rpg.SharedExperts.from_stacked(d["ws1"], d["ws3"], d["ws2"])
        rows = rpg.DenseRows(T, mt, dev)
        buf["hs"] = torch.empty((rows.m_cap, shared.w1.shape[1]), dtype=tdt, device=dev)
        buf["ys"] = torch.empty((rows.m_cap, D), dtype=tdt, device=dev)
    routed = "wg" in d
    stream = torch.cuda.current_stream()
    marks = ["route", "permute", "fc1", "fc2", "shared", "combine"]
    overlap = shared is not None and args.shared_overlap != "none"
    if overlap:
        side = torch.cuda.Stream(device=dev)          # default priority
        gws_side = None if args.no_split_k else rpg.grouped_workspace(dev)
        ev_go, ev_sh = torch.cuda.Event(), torch.cuda.Event()

    def shared_gemm(on, ws):
        rpg.moe_grouped_swiglu(d["x"], rows.offsets, rows.tile_expert, shared.w1, shared.w3,
                               shared.w2, mt, m_cap=rows.m_cap, h=buf["hs"], y_perm=buf["ys"],
                               workspace=ws, stream=on, rows_used=T)

    def launch_side():
        ev_go.record(stream)
        side.wait_event(ev_go)
        shared_gemm(side, gws_side)
        ev_sh.record(side)

    def step(ev=None, ends_only=False):
        def mark(i):
            if ev is not None and (not ends_only or i in (0, len(marks))):
                ev[i].record(stream)
        mark(0)
        if overlap and args.shared_overlap == "start":
            launch_side()
        if routed:
            rpg.moe_route(d["x"], d["wg"], k, bias=d.get("bias"), topk_idx=buf["idx"],
                          topk_w=buf["w"], stream=stream)
        if overlap and args.shared_overlap == "after-route":
            launch_side()
        mark(1)
        rpg.moe_permute(d["x"], buf["idx"], E, mt, m_cap=m_cap, out=buf, stream=stream)
        mark(2)
        rpg.moe_grouped_fc1_swiglu(buf["x_perm"], buf["offsets"], buf["tile_expert"], d["w1"],
                                   d["w3"], mt, m_cap, buf["h"], workspace=gws, stream=stream,
                                   counts=buf["counts"])
        mark(3)
        rpg.moe_grouped_fc2(buf["h"], buf["offsets"], buf["tile_expert"], d["w2"], mt, m_cap,
                            buf["y"], workspace=gws, stream=stream, counts=buf["counts"])
        mark(4)
        sh = None
        if shared is not None:
            if overlap:
                stream.wait_event(ev_sh)
            else:
                shared_gemm(stream, gws)
            sh = buf["ys"][:T]
        mark(5)
        rpg.moe_combine(buf["y"], buf["dst_row"], buf["w"], shared=sh, out=buf["out"],
                        m_cap=m_cap, stream=stream)
        mark(6)

    flush = (torch.empty(args.flush_mib * 1024 * 1024 // 4, dtype=torch.float32, device=dev)
             if args.flush_mib > 0 else None)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if int(buf["dev_err"].item()) != 0:
        raise RuntimeError("permute reported expert indices outside [-1, E)")

    # the K timed steps: one event at each end of a step, nothing recorded inside it
    ends = [[HipEvent() for _ in range(len(marks) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        if flush is not None:
            flush.fill_(float(s))          # outside the step's event brackets
        step(ends[s], ends_only=True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_us = [ends[s][0].elapsed_time(ends[s][-1]) * 1e3 for s in range(args.steps)]
    # K more steps with an event between every two stages: the per-stage times (their
    # marked_step agrees with the timed steps within the run-to-run spread)
    events = [[HipEvent() for _ in range(len(marks) + 1)]
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    for s in range(args.steps):
        if flush is not None:
            flush.fill_(float(s))
        step(events[s])
    torch.cuda.synchronize()

    per = {m: [events[s][i].elapsed_time(events[s][i + 1]) * 1e3 for s in range(args.steps)]
           for i, m in enumerate(marks)}
    per["marked_step"] = [events[s][0].elapsed_time(events[s][-1]) * 1e3
                          for s in range(args.steps)]
    per["step"] = step_us
    med = {m: statistics.median(v) for m, v in per.items()}
    avg = {m: statistics.fmean(v) for m, v in per.items()}

    def pct(v, q):
        return float(np.percentile(np.asarray(v), q))

    spread = {m: {"p10": pct(v, 10), "p90": pct(v, 90),
                  "cv": statistics.pstdev(v) / statistics.fmean(v) if statistics.fmean(v) else 0.0}
              for m, v in per.items()}

    graph = None
    if args.graph and not overlap:
        # the same step captured once (its kernels only: every buffer is allocated above)
        # and replayed K times, each between two events, the cache flush outside them; the
        # replayed output must equal the eager step's bit for bit
        # (captured on a stream of its own, which step() then launches on; replayed on the
        # compute stream)
        ref = buf["out"].clone()
        g = torch.cuda.CUDAGraph()
        main_stream, stream = stream, torch.cuda.Stream()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream):
            step()
        stream = main_stream
        gev = [[HipEvent(), HipEvent()] for _ in range(args.steps)]
        torch.cuda.synchronize()
        for s in range(args.steps):
            buf["out"].zero_()
            if flush is not None:
                flush.fill_(float(s))
            gev[s][0].record(stream)
            g.replay()
            gev[s][1].record(stream)
        torch.cuda.synchronize()
        g_us = [gev[s][0].elapsed_time(gev[s][1]) * 1e3 for s in range(args.steps)]
        graph = {"step_us_mean": statistics.fmean(g_us), "step_us_median": statistics.median(g_us),
                 "tokens_per_s": T / (statistics.fmean(g_us) * 1e-6),
                 "matches_eager_bitwise": bool(torch.equal(buf["out"], ref)),
                 "note": "one step captured with torch.cuda.graph on the compute stream and "
                         "replayed; eager `value` is unchanged"}
        del g

    counts = buf["counts"].cpu().numpy().astype(np.int64)
    n_valid = int(counts.sum())
    n_padded = int(buf["offsets"][-1].item())      # rows the GEMMs compute, pad rows included
    s_el = cfg.elem_bytes
    fc1_flop = 4.0 * n_valid * D * F
    fc2_flop = 2.0 * n_valid * D * F
    gemm_tflops = (fc1_flop + fc2_flop) / ((avg["fc1"] + avg["fc2"]) * 1e-6) / 1e12
    perm_bytes = (T + n_valid) * D * s_el
    comb_bytes = (n_valid + T + (T if shared is not None else 0)) * D * s_el
    perm_gbps = perm_bytes / (avg["permute"] * 1e-6) / 1e9
    comb_gbps = comb_bytes / (avg["combine"] * 1e-6) / 1e9
    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
    fc1_tflops = fc1_flop / (avg["fc1"] * 1e-6) / 1e12
    fc2_tflops = fc2_flop / (avg["fc2"] * 1e-6) / 1e12
    ms_per_step = avg["step"] * 1e-3
    fc1_traffic, fc1_traffic_note = traffic("fc1", cfg.name)
    rec = {
        "metric": METRIC,
        "value": T / (avg["step"] * 1e-6),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded numpy PCG64 draws; Gaussian inputs and weights)",
        "config": {"workload": cfg.name, "T": T, "D": D, "F": F, "E": E, "k": k, "m_tile": mt,
                   "n_shared": cfg.n_shared, "F_shared": cfg.F_shared,
                   "routing": cfg.routing, "split_k_tail": gws is not None,
                   "shared_overlap": args.shared_overlap if shared is not None else None},
        "roofline": {"kernel": "grouped fc1 + silu(a)*b (%s)" % fc1_kernel_name(E, m_cap),
                     "bound": "mfma",
                     "achieved": fc1_tflops, "peak": peak, "unit": "TFLOP/s",
                     "frac": fc1_tflops / peak, "traffic": fc1_traffic,
                     "traffic_unit": "bytes per launch", "traffic_note": fc1_traffic_note,
                     "algorithmic_flop_per_launch": fc1_flop, "avg_launch_us": avg["fc1"]},
        "grouped_gemm_tflops": gemm_tflops,
        "grouped_gemm_frac_bf16_peak": gemm_tflops / peak,
        "fc1_tflops": fc1_tflops, "fc1_frac_bf16_peak": fc1_tflops / peak,
        "fc2_tflops": fc2_tflops, "fc2_frac_bf16_peak": fc2_tflops / peak,
        "route_us": avg["route"] if routed else None,
        "padded": {"rows": n_padded, "fc1_tflops": fc1_tflops * n_padded / max(n_valid, 1),
                   "grouped_gemm_tflops": gemm_tflops * n_padded / max(n_valid, 1),
                   "note": "the same times with pad rows counted as work"},
        "permute_GBps": perm_gbps, "permute_frac_hbm": perm_gbps / PEAK_HBM_GBPS,
        "combine_GBps": comb_gbps, "combine_frac_hbm": comb_gbps / PEAK_HBM_GBPS,
        "stage_us_median": med, "stage_us_mean": avg, "stage_us_spread": spread,
        "timing": {"value_from": "mean of the K steps' durations, each between two HIP events "
                                 "on the compute stream at the step's ends (nothing recorded "
                                 "inside the step)",
                   "stages_from": "K further steps with an event between every two stages "
                                  "(stage_us_*; marked_step is their whole-step mean)",
                   "events": "hipEventCreateWithFlags(hipEventDisableSystemFence): timing only, "
                             "no cache writeback or invalidate at a stage boundary",
                   "cache_flush_MiB_between_steps": args.flush_mib,
                   "wall_ms_per_step_incl_flush": wall * 1e3 / args.steps},
        "assignments": n_valid,
        "expert_rows_min_max": [int(counts.min()), int(counts.max())],
        "cpu_baseline": None,
    }
    if graph is not None:
        rec["graph"] = graph
    if headline and not args.no_backward:
        rec["backward"] = bench_backward(args, cfg, d, buf, shared, gws, flush, n_valid)
    if headline and not args.no_fp8 and cfg.dtype == "bf16" and D % 128 == 0:
        rec["fp8_payload"] = bench_fp8(args, cfg, d, buf, shared, gws, flush, n_valid)
    return rec


def bench_masked(args, cfg, d, inp) -> dict:
    """A decode step on the masked layout: route -> masked permute (slabs of cap rows per
    expert) -> masked grouped SwiGLU [-> shared experts] -> combine, timed like the
    contiguous step. The grouped GEMM of a decode batch streams every active expert's
    weights for a few rows, so its roofline is HBM. The same step on the contiguous
    layout (segments padded to the M tile) is timed next to it."""
    import torch

    import routing_permute_grouped_amd as rpg

    T, D, F, E, k, cap, mt = cfg.T, cfg.D, cfg.F, cfg.E, cfg.k, cfg.cap, cfg.m_tile
    dev = d["x"].device
    tdt = d["x"].dtype
    i32 = dict(dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    gws = None if args.no_split_k else rpg.grouped_workspace(dev)
    buf = {"idx": torch.empty((T, k), **i32), "w": torch.empty((T, k), dtype=torch.float32,
                                                                device=dev),
           "x_masked": torch.empty((E * cap, D), dtype=tdt, device=dev),
           "h": torch.empty((E * cap, F), dtype=tdt, device=dev),
           "y": torch.empty((E * cap, D), dtype=tdt, device=dev),
           "out": torch.empty((T, D), dtype=tdt, device=dev)}
    m_cap = rpg.moe_capacity(T, k, E, mt)
    cbuf = {"x_perm": torch.empty((m_cap, D), dtype=tdt, device=dev),
            "h": torch.empty((m_cap, F), dtype=tdt, device=dev),
            "y": torch.empty((m_cap, D), dtype=tdt, device=dev)}
    shared = None
    if cfg.n_shared:
        shared = rpg.SharedExperts.from_stacked(d["ws1"], d["ws3"], d["ws2"])
        rows = rpg.DenseRows(T, mt, dev)
        buf["hs"] = torch.empty((rows.m_cap, shared.w1.shape[1]), dtype=tdt, device=dev)
        buf["ys"] = torch.empty((rows.m_cap, D), dtype=tdt, device=dev)
    marks = ["route", "permute", "gemm", "shared", "combine"]
    overlap = shared is not None and args.shared_overlap != "none"
    if overlap:
        side = torch.cuda.Stream(device=dev)          # default priority
        gws_side = None if args.no_split_k else rpg.grouped_workspace(dev)
        ev_go, ev_sh = torch.cuda.Event(), torch.cuda.Event()

    def shared_gemm(on, ws):
        rpg.moe_grouped_swiglu(d["x"], rows.offsets, rows.tile_expert, shared.w1, shared.w3,
                               shared.w2, mt, m_cap=rows.m_cap, h=buf["hs"], y_perm=buf["ys"],
                               workspace=ws, stream=on, rows_used=T)

    def launch_side():
        ev_go.record(stream)
        side.wait_event(ev_go)
        shared_gemm(side, gws_side)
        ev_sh.record(side)

    def step(ev=None, contiguous=False, ends_only=False):
        def mark(i):
            if ev is not None and (not ends_only or i in (0, len(marks))):
                ev[i].record(stream)
        mark(0)
        if overlap and args.shared_overlap == "start":
            launch_side()
        rpg.moe_route(d["x"], d["wg"], k, bias=d.get("bias"), topk_idx=buf["idx"],
                      topk_w=buf["w"], stream=stream)
        if overlap and args.shared_overlap == "after-route":
            launch_side()
        mark(1)
        if contiguous:
            p = rpg.moe_permute(d["x"], buf["idx"], E, mt, m_cap=m_cap, out=cbuf, stream=stream)
            cbuf.update(p)   # reuse the metadata buffers from the first call on
            mark(2)
            rpg.moe_grouped_swiglu(p["x_perm"], p["offsets"], p["tile_expert"], d["w1"], d["w3"],
                                   d["w2"], mt, m_cap=m_cap, h=cbuf["h"], y_perm=cbuf["y"],
                                   workspace=gws, stream=stream)
            y, mc = cbuf["y"], m_cap
        else:
            p = rpg.moe_permute_masked(d["x"], buf["idx"], E, cap, out=buf, stream=stream)
            buf.update(p)
            mark(2)
            rpg.moe_grouped_swiglu_masked(p["x_masked"], p["counts"], d["w1"], d["w3"], d["w2"],
                                          cap, h=buf["h"], y=buf["y"], workspace=gws,
                                          stream=stream)
            y, mc = buf["y"], E * cap
        buf["p"] = p
        mark(3)
        sh = None
        if shared is not None:
            if overlap:
                stream.wait_event(ev_sh)
            else:
                shared_gemm(stream, gws)
            sh = buf["ys"][:T]
        mark(4)
        rpg.moe_combine(y, p["dst_row"], buf["w"], shared=sh, out=buf["out"], m_cap=mc,
                        stream=stream)
        mark(5)

    flush = (torch.empty(args.flush_mib * 1024 * 1024 // 4, dtype=torch.float32, device=dev)
             if args.flush_mib > 0 else None)

    def timed(contiguous):
        for _ in range(args.warmup):
            step(contiguous=contiguous)
        torch.cuda.synchronize()
        # the K timed steps with events at their ends only, then K with stage markers
        ends = [[HipEvent() for _ in range(len(marks) + 1)] for _ in range(args.steps)]
        for s_ in range(args.steps):
            if flush is not None:
                flush.fill_(float(s_))
            step(ends[s_], contiguous, ends_only=True)
        events = [[HipEvent() for _ in range(len(marks) + 1)]
                  for _ in range(args.steps)]
        for s_ in range(args.steps):
            if flush is not None:
                flush.fill_(float(s_))
            step(events[s_], contiguous)
        torch.cuda.synchronize()
        per = {m: [events[s_][i].elapsed_time(events[s_][i + 1]) * 1e3
                   for s_ in range(args.steps)] for i, m in enumerate(marks)}
        per["marked_step"] = [events[s_][0].elapsed_time(events[s_][-1]) * 1e3
                              for s_ in range(args.steps)]
        per["step"] = [ends[s_][0].elapsed_time(ends[s_][-1]) * 1e3
                       for s_ in range(args.steps)]
        return ({m: statistics.fmean(v) for m, v in per.items()},
                {m: statistics.median(v) for m, v in per.items()})

    avg, med = timed(False)
    if int(buf["p"]["dev_err"].item()) != 0:
        raise RuntimeError("masked permute flagged bad indices or dropped slots")
    counts = buf["p"]["counts"].cpu().numpy().astype(np.int64)
    cavg, _ = timed(True)
    n_valid = int(counts.sum())
    active = int((counts > 0).sum())
    s_el = cfg.elem_bytes
    w_bytes = active * 3.0 * D * F * s_el
    act_bytes = n_valid * (2.0 * D + 2.0 * F) * s_el
    gemm_bytes = w_bytes + act_bytes
    gbps = gemm_bytes / (avg["gemm"] * 1e-6) / 1e9
    flop = 6.0 * n_valid * D * F
    return {
        "metric": METRIC, "value": T / (avg["step"] * 1e-6), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": avg["step"] * 1e-3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype,
        "data": "synthetic (seeded numpy PCG64 draws; Gaussian inputs and weights)",
        "config": {"workload": cfg.name, "T": T, "D": D, "F": F, "E": E, "k": k,
                   "layout": "masked", "cap": cap, "n_shared": cfg.n_shared,
                   "shared_overlap": args.shared_overlap if shared is not None else None,
                   "F_shared": cfg.F_shared, "split_k_tail": gws is not None},
        "roofline": {"kernel": "grouped fc1 + fc2 on the masked layout (dec_kernel<fc1>, "
                               "<fc2> for bf16 slabs of at most 128 rows, else "
                               "gg_bf16_kernel)", "bound": "hbm",
                     "achieved": gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": gbps / PEAK_HBM_GBPS,
                     "traffic": traffic("masked", cfg.name)[0],
                     "traffic_unit": "bytes per step (fc1 + fc2 launches)",
                     "traffic_note": traffic("masked", cfg.name)[1],
                     "algorithmic_bytes": gemm_bytes,
                     "note": "active experts' w1, w3, w2 once plus the valid rows' x, h "
                             "(written and read) and y"},
        "grouped_gemm_tflops": flop / (avg["gemm"] * 1e-6) / 1e12,
        "stage_us_mean": avg, "stage_us_median": med,
        "timing": {"value_from": "mean of the K steps' durations between HIP events at the "
                                 "step's ends (nothing recorded inside the step)",
                   "stages_from": "K further steps with an event between every two stages",
                   "cache_flush_MiB_between_steps": args.flush_mib},
        "contiguous_layout": {"m_tile": mt, "stage_us_mean": cavg,
                              "ms_per_step": cavg["step"] * 1e-3},
        "assignments": n_valid, "active_experts": active,
        "expert_rows_min_max": [int(counts.min()), int(counts.max())],
        "cpu_baseline": None,
    }


PEAK_FP8_TFLOPS = 5033.2     # MI355X dense fp8 MFMA (AMD spec)


def bench_fp8(args, cfg, d, buf, shared, gws, flush, n_valid) -> dict:
    """The same step with the FP8 payload: route -> MX-quantize x -> permute codes and
    scales -> fc1 on the scaled-FP8 MFMA -> fc2 (bf16) [-> shared experts] -> combine.
    w1 and w3 are quantized once, outside the timed steps. Also reports how far its output
    lies from the bf16 step's."""
    import torch

    import routing_permute_grouped_amd as rpg

    T, D, F, E, k, mt = cfg.T, cfg.D, cfg.F, cfg.E, cfg.k, cfg.m_tile
    dev = d["x"].device
    stream = torch.cuda.current_stream()
    m_cap = buf["x_perm"].shape[0]
    mw = rpg.MxWeights.quantize(d["w1"], d["w3"])
    u8 = dict(dtype=torch.uint8, device=dev)
    fb = {"xq": torch.empty((T, D), **u8), "xs": torch.empty((T, D // 32), **u8),
          "xq_perm": torch.empty((m_cap, D), **u8), "xs_perm": torch.empty((D // 128, m_cap, 4), **u8),
          "out": torch.empty_like(buf["out"])}
    for n in ("counts", "offsets", "dst_row", "src_row", "tile_expert", "dev_err", "workspace"):
        fb[n] = torch.empty_like(buf[n])
    marks = ["route", "quantize", "permute", "fc1", "fc2", "shared", "combine"]
    routed = "wg" in d

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record(stream)
        mark(0)
        if routed:
            rpg.moe_route(d["x"], d["wg"], k, bias=d.get("bias"), topk_idx=buf["idx"],
                          topk_w=buf["w"], stream=stream)
        mark(1)
        rpg.moe_quantize_mxfp8(d["x"], q=fb["xq"], scales=fb["xs"], stream=stream)
        mark(2)
        rpg.moe_permute_mxfp8(fb["xq"], fb["xs"], buf["idx"], E, mt, m_cap=m_cap, out=fb,
                              stream=stream)
        mark(3)
        rpg.moe_grouped_fc1_swiglu_mxfp8(fb["xq_perm"], fb["xs_perm"], fb["offsets"],
                                         fb["tile_expert"], mw.w1q, mw.w1s, mw.w3q, mw.w3s, mt,
                                         m_cap, h=buf["h"], workspace=gws, stream=stream,
                                         counts=fb["counts"])
        mark(4)
        rpg.moe_grouped_fc2(buf["h"], fb["offsets"], fb["tile_expert"], d["w2"], mt, m_cap,
                            buf["y"], workspace=gws, stream=stream, counts=fb["counts"])
        mark(5)
        sh = None
        if shared is not None:
            rows = rpg.DenseRows(T, mt, dev)
            rpg.moe_grouped_swiglu(d["x"], rows.offsets, rows.tile_expert, shared.w1, shared.w3,
                                   shared.w2, mt, m_cap=rows.m_cap, h=buf["hs"],
                                   y_perm=buf["ys"], workspace=gws, stream=stream, rows_used=T)
            sh = buf["ys"][:T]
        mark(6)
        rpg.moe_combine(buf["y"], fb["dst_row"], buf["w"], shared=sh, out=fb["out"],
                        m_cap=m_cap, stream=stream)
        mark(7)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[HipEvent() for _ in range(len(marks) + 1)]
              for _ in range(args.steps)]
    for s_ in range(args.steps):
        if flush is not None:
            flush.fill_(float(s_))
        step(events[s_])
    torch.cuda.synchronize()
    per = {m: [events[s_][i].elapsed_time(events[s_][i + 1]) * 1e3 for s_ in range(args.steps)]
           for i, m in enumerate(marks)}
    per["step"] = [events[s_][0].elapsed_time(events[s_][-1]) * 1e3 for s_ in range(args.steps)]
    avg = {m: statistics.fmean(v) for m, v in per.items()}
    fc1_flop = 4.0 * n_valid * D * F
    fc1_tf = fc1_flop / (avg["fc1"] * 1e-6) / 1e12
    ref = buf["out"].float()
    dev_out = (fb["out"].float() - ref).abs().max().item() / ref.abs().max().item()
    return {
        "tokens_per_s": T / (avg["step"] * 1e-6), "ms_per_step": avg["step"] * 1e-3,
        "fc1": {"kernel": "grouped fc1 + silu(a)*b on MX e4m3 (gg_bf16_kernel<kFc1, MX>)",
                "achieved_tflops": fc1_tf, "peak_fp8_tflops": PEAK_FP8_TFLOPS,
                "frac_fp8_peak": fc1_tf / PEAK_FP8_TFLOPS,
                "frac_bf16_peak": fc1_tf / PEAK_BF16_TFLOPS,
                "traffic": traffic("fp8_fc1", cfg.name)[0],
                "traffic_unit": "bytes per launch",
                "traffic_note": traffic("fp8_fc1", cfg.name)[1]},
        "stage_us_mean": avg,
        "out_rel_diff_vs_bf16_step": dev_out,
        "note": "x quantized per token (32-value blocks, power-of-two scales, no saturation); "
                "w1, w3 quantized once; fc2, shared experts and combine in bf16",
    }


def bench_backward(args, cfg, d, buf, shared, gws, flush, n_valid) -> dict:
    """Time the layer's backward for a seeded output gradient, every buffer allocated
    beforehand: combine backward -> dgrad (dh -> [da | db], then dX) -> wgrad ([dW1 | dW3],
    dW2) [-> the shared experts' backward] -> unpermute. The forward is run once before
    (untimed) with fc1 keeping [a | b]."""
    import torch

    import routing_permute_grouped_amd as rpg
    import workloads as W

    T, D, F, E, k, mt = cfg.T, cfg.D, cfg.F, cfg.E, cfg.k, cfg.m_tile
    dev = d["x"].device
    tdt = d["x"].dtype
    stream = torch.cuda.current_stream()
    m_cap = buf["x_perm"].shape[0]

    def em(*shape, dtype=tdt):
        return torch.empty(shape, dtype=dtype, device=dev)

    dout_np = W.output_grad(cfg, seed=1)
    dout = (torch.from_numpy(dout_np.view(np.int16)).to(dev).view(torch.bfloat16)
            if dout_np.dtype == np.uint16 else torch.from_numpy(dout_np).to(dev))
    f32 = torch.float32
    b = {"ab": em(m_cap, 2 * F), "dy": em(m_cap, D), "dtw": em(T, k, dtype=f32),
         "dab": em(m_cap, 2 * F), "dX": em(m_cap, D), "dw1": em(E, F, D, dtype=f32),
         "dw3": em(E, F, D, dtype=f32), "dw2": em(E, D, F, dtype=f32), "dx": em(T, D)}
    offs, te = buf["offsets"], buf["tile_expert"]
    # forward once more, keeping fc1's pre-activations (routing/permute as in the timed run)
    cnt = buf["counts"]
    rpg.moe_grouped_fc1_swiglu(buf["x_perm"], offs, te, d["w1"], d["w3"], mt, m_cap, buf["h"],
                               ab=b["ab"], workspace=gws, counts=cnt)
    rpg.moe_grouped_fc2(buf["h"], offs, te, d["w2"], mt, m_cap, buf["y"], workspace=gws,
                        counts=cnt)
    if shared is not None:
        rows = rpg.DenseRows(T, mt, dev)
        SF = shared.w1.shape[1]
        b.update(s_h=em(rows.m_cap, SF), s_ab=em(rows.m_cap, 2 * SF),
                 s_dab=em(rows.m_cap, 2 * SF), s_dX=em(rows.m_cap, D),
                 s_dw1=em(1, SF, D, dtype=f32), s_dw3=em(1, SF, D, dtype=f32),
                 s_dw2=em(1, D, SF, dtype=f32))
        rpg.moe_grouped_fc1_swiglu(d["x"], rows.offsets, rows.tile_expert, shared.w1, shared.w3,
                                   mt, rows.m_cap, b["s_h"], ab=b["s_ab"], workspace=gws,
                                   rows_used=T)

    def experts_bwd(dy, xr, ab, h, o, tt, w1, w3, w2, mcap, pre, ru=None, c=None):
        Fx = w1.shape[1]
        rpg.moe_grouped_dgrad_swiglu(dy, o, tt, w2, ab, mt, mcap, dab=b[pre + "dab"],
                                     workspace=gws, stream=stream, rows_used=ru, counts=c)
        mark()
        rpg.moe_grouped_dgrad_fc1(b[pre + "dab"], o, tt, w1, w3, mt, mcap, dx_perm=b[pre + "dX"],
                                  workspace=gws, stream=stream, rows_used=ru, counts=c)
        mark()
        rpg.moe_grouped_wgrad(b[pre + "dab"], xr, o, mt, mcap, NS=Fx, out_lo=b[pre + "dw1"],
                              out_hi=b[pre + "dw3"], stream=stream, rows_used=ru, counts=c)
        mark()
        rpg.moe_grouped_wgrad(dy, h, o, mt, mcap, NS=D, out_lo=b[pre + "dw2"], stream=stream,
                              rows_used=ru, counts=c)
        mark()

    marks = ["combine_bwd", "dgrad_fc2", "dgrad_fc1", "wgrad_fc1", "wgrad_fc2"]
    if shared is not None:
        marks += ["s_dgrad_fc2", "s_dgrad_fc1", "s_wgrad_fc1", "s_wgrad_fc2"]
    marks += ["unpermute"]
    cur = {"ev": None, "i": 0}

    def mark():
        if cur["ev"] is not None:
            cur["ev"][cur["i"]].record(stream)
        cur["i"] += 1

    def step(ev=None):
        cur["ev"], cur["i"] = ev, 0
        mark()
        rpg.moe_combine_backward(dout, buf["y"], buf["src_row"], offs, buf["dst_row"], buf["w"],
                                 m_cap=m_cap, dy_perm=b["dy"], dtopk_w=b["dtw"], stream=stream)
        mark()
        experts_bwd(b["dy"], buf["x_perm"], b["ab"], buf["h"], offs, te, d["w1"], d["w3"],
                    d["w2"], m_cap, "", c=cnt)
        sh = None
        if shared is not None:
            experts_bwd(dout, d["x"], b["s_ab"], b["s_h"], rows.offsets, rows.tile_expert,
                        shared.w1, shared.w3, shared.w2, rows.m_cap, "s_", T)
            sh = b["s_dX"][:T]
        rpg.moe_combine(b["dX"], buf["dst_row"], None, shared=sh, out=b["dx"], m_cap=m_cap,
                        stream=stream)
        mark()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[HipEvent() for _ in range(len(marks) + 1)]
              for _ in range(args.steps)]
    for s_ in range(args.steps):
        if flush is not None:
            flush.fill_(float(s_))
        step(events[s_])
    torch.cuda.synchronize()
    per = {m: [events[s_][i].elapsed_time(events[s_][i + 1]) * 1e3 for s_ in range(args.steps)]
           for i, m in enumerate(marks)}
    per["step"] = [events[s_][0].elapsed_time(events[s_][-1]) * 1e3 for s_ in range(args.steps)]
    avg = {m: statistics.fmean(v) for m, v in per.items()}
    med = {m: statistics.median(v) for m, v in per.items()}
    ndf = float(n_valid) * D * F
    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS

    def tf(flop, *stages):
        t = sum(avg[m] for m in stages)
        return flop / (t * 1e-6) / 1e12

    gemm_stages = ["dgrad_fc2", "dgrad_fc1", "wgrad_fc1", "wgrad_fc2"]
    routed_flop = 12.0 * ndf
    wg1 = tf(4 * ndf, "wgrad_fc1")
    out = {
        "tokens_per_s": T / (avg["step"] * 1e-6),
        "ms_per_step": avg["step"] * 1e-3,
        "algorithmic_flop": {"routed": routed_flop,
                             "shared": 12.0 * T * D * cfg.n_shared * cfg.F_shared},
        "kernels_tflops": {"dgrad_fc2 (dh -> [da|db])": tf(2 * ndf, "dgrad_fc2"),
                           "dgrad_fc1 (dX)": tf(4 * ndf, "dgrad_fc1"),
                           "wgrad_fc1 ([dW1|dW3])": tf(4 * ndf, "wgrad_fc1"),
                           "wgrad_fc2 (dW2)": tf(2 * ndf, "wgrad_fc2")},
        "roofline": {"kernel": "k-grouped wgrad of fc1, [dW1 | dW3] (wg_bf16_kernel)",
                     "bound": "mfma", "achieved": wg1, "peak": peak, "unit": "TFLOP/s",
                     "frac": wg1 / peak, "traffic": traffic("wgrad_fc1", cfg.name)[0],
                     "traffic_unit": "bytes per launch",
                     "traffic_note": traffic("wgrad_fc1", cfg.name)[1],
                     "algorithmic_flop_per_launch": 4 * ndf, "avg_launch_us": avg["wgrad_fc1"]},
        "grouped_gemm_tflops": tf(routed_flop, *gemm_stages),
        "grouped_gemm_frac_bf16_peak": tf(routed_flop, *gemm_stages) / peak,
        "stage_us_mean": avg, "stage_us_median": med,
        "note": "algorithmic FLOP: 12 D F per routed assignment (dgrad 6 + wgrad 6); "
                "weight gradients are float32",
    }
    return out


if __name__ == "__main__":
    main()
