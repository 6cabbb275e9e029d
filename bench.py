#!/usr/bin/env python3
"""Throughput of exact tiled attention (BF16) on one MI355X.

One step = the whole hot path on one batch: fa_fwd (O, LSE) then fa_bwd (dQ, dK,
dV; deterministic dQ by default, --atomic for atomic dQ) on the causal B=2, H=16,
S=8192, d=128 workload (synthetic normal inputs, already resident in HBM).  Throughput counts algorithmic FLOP:
4*d per visible (query, key) pair forward and 10*d backward, causal pairs only.

Prints one JSON line.  Per-kernel average durations come from HIP events on the
stream the library launches on (torch's current stream); the roofline object
describes the kernel with the largest share of the step.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense BF16 MFMA, AMD's published 2.5 PFLOP/s (256 CU x 2.4 GHz x 4096
                            # FLOP/clk/CU = 2516.6 before rounding)
PEAK_HBM_GBS = 8000.0
WORKLOAD = "headline"       # causal B=2 H=16 S=8192 d=128
COPY_BYTES = 1 << 30        # calibration copy: 1 GiB read + 1 GiB written
BWD_SEED_CONFIG = "c5"      # same shape with dO


def log(*a):
    print(*a, file=sys.stderr, flush=True)


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "attn_causal_B2_H16_S8192_d128_hbm_traffic.md")


def recorded_traffic(phase: str):
    """HBM-side bytes per launch (read + written) of a kernel, from the committed
    counter summary (FETCH_SIZE / WRITE_SIZE scaled by a copy of known size); None
    when there is no record or the kernel's sources changed since it was taken."""
    import hashlib
    try:
        lines = open(TRAFFIC_PROFILE).read().splitlines()
    except OSError:
        return None
    for ln in lines:
        if not ln.startswith("traffic-record: "):
            continue
        rec = json.loads(ln[len("traffic-record: "):])
        if rec["phase"] != phase:
            continue
        h = hashlib.sha256()
        for f in rec["sources"]:
            h.update(open(os.path.join(ROOT, "tiled_exact_attention_bf16_amd", "csrc", f), "rb").read())
        if h.hexdigest() != rec["source_sha256"]:
            return None
        return int(rec["read_bytes"]) + int(rec["write_bytes"])
    return None


class ClockSampler:
    """Shader clock while the kernels run: amdsmi's current GFX clock of each of the
    GPU's XCDs (gpu metrics), polled every 5 ms by a background thread; each new
    reading (the amdgpu kernel driver refreshes them far less often than that) counts
    once, and readings of an idle GPU (below 500 MHz, deep sleep) are dropped.  None without
    amdsmi."""

    def __init__(self):
        import threading
        self.mhz = []
        self._stop = threading.Event()
        self._t = threading.Thread(target=self._run, daemon=True)
        self.ok = False
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self._smi = amdsmi
            self._h = amdsmi.amdsmi_get_processor_handles()[0]
            self.ok = True
        except Exception:  # pragma: no cover
            self.ok = False

    def _run(self):
        last = None
        while not self._stop.is_set():
            try:
                cur = self._smi.amdsmi_get_gpu_metrics_info(self._h).get("current_gfxclks")
                vals = [float(x) for x in cur if isinstance(x, (int, float)) and 0 < x < 10000]
                if vals and vals != last:
                    last = vals
                    if min(vals) >= 500:
                        self.mhz.append(sum(vals) / len(vals))
            except Exception:
                pass
            time.sleep(0.005)

    def __enter__(self):
        if self.ok:
            self._t.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self.ok:
            self._t.join()

    def summary(self):
        if not self.mhz:
            return None
        return {"mean_mhz": round(float(np.mean(self.mhz)), 1), "min_mhz": round(min(self.mhz), 1),
                "max_mhz": round(max(self.mhz), 1), "samples": len(self.mhz),
                "source": "amdsmi current_gfxclks (mean over XCDs), each new reading from warm-up until "
                          "three busy readings arrived while the same step kept running after the timed region"}


def at_clock(clock, step_tf: float, fwd_tf: float, bwd_tf: float):
    """The same rates against the MFMA peak at the shader clock measured during the run
    (the 2.5 PFLOP/s figure assumes 2.4 GHz; these kernels run the chip well below)."""
    if not clock:
        return None
    peak = PEAK_BF16_TFLOPS * clock["mean_mhz"] / 2400.0
    return {"peak_tflops": round(peak, 1), "frac_of_peak": round(step_tf / peak, 4),
            "fwd_frac_of_peak": round(fwd_tf / peak, 4), "bwd_frac_of_peak": round(bwd_tf / peak, 4)}


def cpu_model() -> str:
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp, budget_s: float = 12.0, max_heads: int = 8):
    """The fp64 oracle (as it stands) on a bounded sample of the same workload:
    forward then backward of whole (sequence, head) pairs, until ``budget_s``."""
    from oracle import attention as OA
    from tiled_exact_attention_bf16_amd import inputs as I
    from tiled_exact_attention_bf16_amd import workload as W
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    done, t_total, flop = 0, 0.0, 0
    pairs = [(b, h) for b in range(inp.batch) for h in range(inp.num_heads)]
    for b, h in pairs[:max_heads]:
        q, k, v, do = (I.bf16_bits_to_f64(inp.sequence(b, t)[:, h]) for t in ("q", "k", "v", "do"))
        t0 = time.perf_counter()
        OA.head_forward(q, k, v, inp.scale, inp.causal)
        OA.head_backward(q, k, v, do, inp.scale, inp.causal)
        t_total += time.perf_counter() - t0
        s = q.shape[0]
        flop += W.fwd_flops([s], [s], 1, q.shape[1], inp.causal) + W.bwd_flops([s], [s], 1, q.shape[1], inp.causal)
        done += 1
        if t_total >= budget_s:
            break
    return {"value": round(flop / t_total / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"fp64 numpy forward+backward of {done} whole (sequence, head) pairs of the "
                      f"{inp.q.shape[1]}-token causal workload, {t_total:.1f} s"}


def time_all_configs(deterministic: bool, warmup: int = 10, iters: int = 50):
    """Forward and backward TFLOP/s of every named workload: median and min over
    `iters` timed calls (HIP events on the library's stream) after `warmup` calls."""
    import torch
    from tiled_exact_attention_bf16_amd import attention as FA
    from tiled_exact_attention_bf16_amd import inputs as I
    from tiled_exact_attention_bf16_amd import workload as W
    res = {}
    dev = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()
    for name in ("c1", "c2", "c2_causal", "c3", "c4", "headline", "c5"):
        inp = I.make_inputs(name)
        log(f"[bench] config {name}")
        q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
        if inp.do is not None:
            do = dev(inp.do)
        else:  # timing only: dO values do not change the work
            g = torch.Generator(device="cuda").manual_seed(inp.seed + 1000)
            do = torch.randn(q.shape, generator=g, device="cuda").to(torch.bfloat16)
        cu = torch.from_numpy(inp.cu_seqlens).cuda() if inp.varlen else None
        mx = inp.max_seqlen() if inp.varlen else None
        lens = [int(x) for x in inp.seqlens()]
        f_fwd = W.fwd_flops(lens, lens, inp.num_heads, q.shape[-1], inp.causal)
        f_bwd = W.bwd_flops(lens, lens, inp.num_heads, q.shape[-1], inp.causal)
        ws_f = FA.fwd_workspace(q, k, v, inp.scale, inp.causal, cu_seqlens_q=cu, max_seqlen_q=mx)
        o, lse = FA.fwd(q, k, v, inp.scale, inp.causal, cu_seqlens_q=cu, max_seqlen_q=mx, workspace=ws_f)
        dq, dk, dv = (torch.empty(t.shape, dtype=torch.float32, device="cuda") for t in (q, k, v))
        ws_b = torch.empty(2 << 30, dtype=torch.uint8, device="cuda")  # atomic c4: 1.07 GB accumulator
        run = {"fwd": lambda: FA.fwd(q, k, v, inp.scale, inp.causal, cu_seqlens_q=cu, max_seqlen_q=mx,
                                     out=o, lse=lse, workspace=ws_f),
               "bwd": lambda: FA.bwd(do, q, k, v, o, lse, inp.scale, inp.causal, cu_seqlens_q=cu,
                                     max_seqlen_q=mx, deterministic=deterministic, dq=dq, dk=dk, dv=dv,
                                     workspace=ws_b),
               "bwd_" + ("atomic" if deterministic else "deterministic"):
                   lambda: FA.bwd(do, q, k, v, o, lse, inp.scale, inp.causal, cu_seqlens_q=cu,
                                  max_seqlen_q=mx, deterministic=not deterministic, dq=dq, dk=dk, dv=dv,
                                  workspace=ws_b)}
        row = {}
        # the 4096-token workloads (K+V 128 MiB) fit in the 256 MB last-level cache: time
        # them also with a 512 MiB scratch write between calls (outside the timed region)
        flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda") if name in ("c2", "c2_causal") else None
        for ph, fn in run.items():
            for _ in range(warmup):
                fn()
            for flushed in ((False, True) if flush is not None else (False,)):
                ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                      for _ in range(iters)]
                for i, (a, b) in enumerate(ev):
                    if flushed:
                        flush.fill_(i & 0xFF)
                    a.record()
                    fn()
                    b.record()
                torch.cuda.synchronize()
                ms = np.array([a.elapsed_time(b) for a, b in ev])
                flop = f_fwd if ph == "fwd" else f_bwd
                row[ph + ("_cache_flushed" if flushed else "")] = {
                    "median_ms": round(float(np.median(ms)), 4), "min_ms": round(float(ms.min()), 4),
                    "tflops_median": round(flop / (np.median(ms) * 1e-3) / 1e12, 2),
                    "tflops_max": round(flop / (ms.min() * 1e-3) / 1e12, 2)}
        res[name] = row
        del flush
        del q, k, v, do, o, lse, dq, dk, dv, ws_f, ws_b
        torch.cuda.empty_cache()
    return res


def run_workload(name: str, steps: int, warmup: int, deterministic: bool, tau: int = -1):
    """Forward then backward of one named workload, `steps` times after `warmup` (for
    profiling one workload under rocprofv3); prints per-phase HIP-event averages."""
    import torch
    from tiled_exact_attention_bf16_amd import _lib as L
    from tiled_exact_attention_bf16_amd import attention as FA
    from tiled_exact_attention_bf16_amd import inputs as I
    from tiled_exact_attention_bf16_amd import workload as W
    inp = I.make_inputs(name)
    dev = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    do = dev(inp.do) if inp.do is not None else torch.randn(q.shape, device="cuda").to(torch.bfloat16)
    cu = torch.from_numpy(inp.cu_seqlens).cuda() if inp.varlen else None
    mx = inp.max_seqlen() if inp.varlen else None
    t = FA.Tuning(rescale_threshold_log2=tau)
    ws_f = FA.fwd_workspace(q, k, v, inp.scale, inp.causal, cu_seqlens_q=cu, max_seqlen_q=mx, tuning=t)
    ws_b = torch.empty(2 << 30, dtype=torch.uint8, device="cuda")
    o, lse = FA.fwd(q, k, v, inp.scale, inp.causal, cu_seqlens_q=cu, max_seqlen_q=mx, workspace=ws_f, tuning=t)
    dq, dk, dv = (torch.empty(x.shape, dtype=torch.float32, device="cuda") for x in (q, k, v))
    fns = {"fwd": lambda: FA.fwd(q, k, v, inp.scale, inp.causal, cu_seqlens_q=cu, max_seqlen_q=mx, out=o, lse=lse,
                                 workspace=ws_f, tuning=t),
           "bwd": lambda: FA.bwd(do, q, k, v, o, lse, inp.scale, inp.causal, cu_seqlens_q=cu, max_seqlen_q=mx,
                                 deterministic=deterministic, dq=dq, dk=dk, dv=dv, workspace=ws_b)}
    for _ in range(warmup):
        for fn in fns.values():
            fn()
    ev = {n: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
          for n in fns}
    for i in range(steps):
        for n, fn in fns.items():
            ev[n][i][0].record()
            fn()
            ev[n][i][1].record()
    torch.cuda.synchronize()
    lens = [int(x) for x in inp.seqlens()]
    fl = {"fwd": W.fwd_flops(lens, lens, inp.num_heads, q.shape[-1], inp.causal),
          "bwd": W.bwd_flops(lens, lens, inp.num_heads, q.shape[-1], inp.causal)}
    res = {}
    for n in fns:
        ms = float(np.mean([a.elapsed_time(b) for a, b in ev[n]]))
        res[n] = {"ms": round(ms, 4), "tflops": round(fl[n] / (ms * 1e-3) / 1e12, 2)}
    print(json.dumps({"workload": name, "deterministic": deterministic, "tau": tau, **res}), flush=True)


def time_decode(warmup: int = 10, iters: int = 50):
    """Short queries against a long key sequence (generation with a cache): forward
    time with the key split chosen from the shape and with no split.  Device-side
    normal inputs (values do not change the work); K+V bytes / time is reported
    next to TFLOP/s because these shapes are bound by reading K and V."""
    import torch
    from tiled_exact_attention_bf16_amd import attention as FA
    from tiled_exact_attention_bf16_amd import workload as W
    B, H, D, LK = 4, 16, 128, 16384
    g = torch.Generator(device="cuda").manual_seed(7)
    k = torch.randn((B, LK, H, D), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((B, LK, H, D), generator=g, device="cuda").to(torch.bfloat16)
    res = {}
    for lq in (1, 16, 128):
        q = torch.randn((B, lq, H, D), generator=g, device="cuda").to(torch.bfloat16)
        o = torch.empty_like(q)
        lse = torch.empty((B, H, lq), dtype=torch.float32, device="cuda")
        flop = W.fwd_flops([lq] * B, [LK] * B, H, D, True)
        kv_bytes = 2 * B * LK * H * D * 2
        row = {}
        for label, splits in (("auto_split", -1), ("no_split", 1)):
            t = FA.Tuning(key_splits=splits)
            ws = FA.fwd_workspace(q, k, v, 1.0 / D ** 0.5, True, tuning=t)
            fn = lambda: FA.fwd(q, k, v, 1.0 / D ** 0.5, True, tuning=t, out=o, lse=lse, workspace=ws)
            for _ in range(warmup):
                fn()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
            for a, b in ev:
                a.record()
                fn()
                b.record()
            torch.cuda.synchronize()
            ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
            row[label] = {"median_ms": round(ms, 4), "tflops": round(flop / (ms * 1e-3) / 1e12, 2),
                          "kv_gbs": round(kv_bytes / (ms * 1e-3) / 1e9, 1)}
        res[f"B{B} H{H} d{D} Lq{lq} Lk{LK} causal"] = row
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--atomic", action="store_true",
                    help="time the backward with atomic dQ accumulation (default: the deterministic mode)")
    ap.add_argument("--q-tiles", type=int, default=-1)
    ap.add_argument("--poly", type=int, default=-1)
    ap.add_argument("--tau", type=int, default=-1)
    ap.add_argument("--all-configs", action="store_true",
                    help="also time forward and backward of every named workload (median/min of 50)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the other dQ mode's timing and the clock sampling (short profiled runs)")
    ap.add_argument("--workload", default=None,
                    help="only run forward+backward of this named workload (c1..c5, c2_causal, headline) "
                         "--steps times and print per-phase averages (for profiling)")
    ap.add_argument("--decode-only", action="store_true",
                    help="only time the generation shapes (short queries against 16K keys, with the "
                         "automatic key split and without a split) and print them (for profiling)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also launch a plain device copy of a known size (for scaling HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from tiled_exact_attention_bf16_amd import _lib as L
    from tiled_exact_attention_bf16_amd import attention as FA
    from tiled_exact_attention_bf16_amd import inputs as I
    from tiled_exact_attention_bf16_amd import workload as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    L.lib()  # fail loudly if the HIP library is missing
    if args.workload:
        run_workload(args.workload, args.steps, args.warmup, not args.atomic, args.tau)
        return
    if args.decode_only:
        print(json.dumps({"decode": time_decode()}), flush=True)
        return

    inp = I.make_inputs(BWD_SEED_CONFIG)   # B=2 S=8192 H=16 d=128 causal, with dO
    B, S, H, D = inp.q.shape
    log(f"[bench] workload causal B={B} S={S} H={H} d={D}; uploading")
    dev = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()
    q, k, v, do = dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.do)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device="cuda")
    dq = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    dk = torch.empty(k.shape, dtype=torch.float32, device="cuda")
    dv = torch.empty(v.shape, dtype=torch.float32, device="cuda")
    ws = torch.empty(1 << 28, dtype=torch.uint8, device="cuda")   # >= either mode's workspace (fp32 dQ accumulator)
    tuning = FA.Tuning(args.poly, args.tau, args.q_tiles)
    ws_f = FA.fwd_workspace(q, k, v, inp.scale, True, tuning=tuning)  # the fp16 copy of V
    det = not args.atomic

    def fwd():
        FA.fwd(q, k, v, inp.scale, True, tuning=tuning, out=o, lse=lse, workspace=ws_f)

    def bwd(phases=L.FA_BWD_PHASE_ALL):
        FA.bwd(do, q, k, v, o, lse, inp.scale, True, deterministic=det, dq=dq, dk=dk, dv=dv, workspace=ws,
               phases=phases)

    clk = ClockSampler() if not args.no_extras else None
    if clk is not None:
        clk.__enter__()
    for _ in range(args.warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()

    # per-kernel events on the library's stream (torch's current stream)
    names = ["fwd", "bwd_pre", "bwd_main", "bwd_post"]
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        e = ev[i]
        e[0].record()
        fwd()
        e[1].record()
        bwd(L.FA_BWD_PHASE_PRE)
        e[2].record()
        bwd(L.FA_BWD_PHASE_MAIN)
        e[3].record()
        bwd(L.FA_BWD_PHASE_POST)
        e[4].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # the amdgpu kernel driver refreshes its clock readings only every few hundred ms, and
    # a short timed region can end before one shows the busy clock: keep running the same step
    # outside the timed region until three busy readings have arrived, for at most 4 s
    if clk is not None:
        t1 = time.perf_counter()
        while time.perf_counter() - t1 < 4.0 and len(clk.mhz) < 3:
            fwd()
            bwd()
            torch.cuda.synchronize()
        clk.__exit__(None, None, None)
    if args.copy_calibration:
        # outside the timed region: one copy kernel reading and writing COPY_BYTES
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy calibration: {COPY_BYTES} bytes read and written")
    per = {n: float(np.mean([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(args.steps)]))
           for j, n in enumerate(names)}
    step_ms = float(np.mean([ev[i][0].elapsed_time(ev[i][4]) for i in range(args.steps)]))

    seq = [S] * B
    f_fwd = W.fwd_flops(seq, seq, H, D, True)
    f_bwd = W.bwd_flops(seq, seq, H, D, True)
    fwd_tf = f_fwd / (per["fwd"] * 1e-3) / 1e12
    bwd_ms = per["bwd_pre"] + per["bwd_main"] + per["bwd_post"]
    bwd_tf = f_bwd / (bwd_ms * 1e-3) / 1e12
    # whole-step throughput from the wall clock around the timed steps (the same clock as
    # ms_per_step); the per-kernel events give the breakdown
    value = (f_fwd + f_bwd) / (wall / args.steps) / 1e12
    # algorithmic FLOP per visible pair for each kernel: forward 4d (S, PV); key-block
    # kernel 8d (S, dP, dV, dK) in deterministic mode, 10d with the atomic dQ product;
    # deterministic dQ kernel 2d (dQ; its S and dP are recomputation)
    pairs = W.total_pairs(seq, seq, H, True)
    alg = {"fwd": 4 * D * pairs, "bwd_main": (8 if det else 10) * D * pairs,
           "bwd_post": 2 * D * pairs if det else 0, "bwd_pre": 0}
    dominant = max(("fwd", "bwd_main", "bwd_post"), key=lambda n: per[n])
    achieved = alg[dominant] / (per[dominant] * 1e-3) / 1e12
    kernel_names = {"fwd": "fa::fwd_kernel<128,2,causal>",
                    "bwd_main": "fa::bwd_kv_kernel<128,causal," + ("deterministic>" if det else "atomic>"),
                    "bwd_post": "fa::bwd_dq_kernel<128,causal>" if det else "fa::bwd_post_kernel<128>"}
    out = {
        "metric": "attention fwd/bwd TFLOP/s (BF16, d=128, causal S=8K) and % of MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "causal attention forward+backward, B=2 H=16 S=8192 d=128 (bf16 in, fp32 grads, "
                               + ("deterministic" if det else "atomic") + " dQ)",
                   "global_batch": B, "seq_len": S, "heads": H, "head_dim": D, "causal": True,
                   "parallelism": "single-gpu"},
        "frac_of_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "fwd_tflops": round(fwd_tf, 2),
        "fwd_frac_of_peak": round(fwd_tf / PEAK_BF16_TFLOPS, 4),
        "bwd_tflops": round(bwd_tf, 2),
        "bwd_frac_of_peak": round(bwd_tf / PEAK_BF16_TFLOPS, 4),
        "kernel_ms": {n: round(per[n], 4) for n in names},
        "events_step_ms": round(step_ms, 4),
        "shader_clock": clk.summary() if clk is not None else None,
        "at_measured_clock": at_clock(clk.summary() if clk is not None else None, value, fwd_tf, bwd_tf),
        "roofline": {"bound": "mfma", "kernel": kernel_names[dominant], "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": recorded_traffic(dominant) if det or dominant == "fwd" else None},
    }
    # the other dQ mode of the same backward, outside the timed step (reported beside it)
    other = not det
    if args.no_extras:
        other = None

    def bwd_other(phases):
        FA.bwd(do, q, k, v, o, lse, inp.scale, True, deterministic=other, dq=dq, dk=dk, dv=dv, workspace=ws,
               phases=phases)

    for _ in range(args.warmup if other is not None else 0):
        bwd_other(L.FA_BWD_PHASE_ALL)
    ev2 = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps if other is not None else 0)]
    for i in range(len(ev2)):
        e = ev2[i]
        e[0].record()
        bwd_other(L.FA_BWD_PHASE_PRE)
        e[1].record()
        bwd_other(L.FA_BWD_PHASE_MAIN)
        e[2].record()
        bwd_other(L.FA_BWD_PHASE_POST)
        e[3].record()
    torch.cuda.synchronize()
    if other is not None:
        per2 = {n: float(np.mean([ev2[i][j].elapsed_time(ev2[i][j + 1]) for i in range(args.steps)]))
                for j, n in enumerate(("bwd_pre", "bwd_main", "bwd_post"))}
        ms2 = sum(per2.values())
        out["bwd_" + ("deterministic" if other else "atomic")] = {
            "ms": round(ms2, 4), "tflops": round(f_bwd / (ms2 * 1e-3) / 1e12, 2),
            "kernel_ms": {n: round(x, 4) for n, x in per2.items()}}
    if args.all_configs:
        out["configs"] = time_all_configs(det)
        out["decode"] = time_decode()
    if not args.no_cpu_baseline:
        log("[bench] timing the fp64 oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(inp)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
