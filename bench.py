"""Benchmark: FlashAttention forward throughput on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--dtype bf16|fp16]

A step is one pass of the forward over one batch of synthetic input: phase 1
(plan) and phase 2 (the HIP kernels) of ``libfa_fwd.so``.  Inputs are resident
in GPU memory before the timed region.  The default workload is dense BSND
B=2 S=4096 N=24 D=128 in bf16 with no mask, scale 1/sqrt(128).

Prints one JSON line.  ``value`` is TFLOP/s over the timed steps, counting
4*D FLOP per kept (query, key) pair (2*(D+Dr) + 2*Dv with rope parts), with
kept pairs counted on 128x128 blocks as the workloads' accounting asks.
``roofline`` prices the forward kernel's average duration, measured with HIP
events on the launch stream during the timed region, against the MI355X dense
matrix peak.  ``cpu_baseline`` times the CPU float64 oracle on a bounded
sample of the same workload.

After the timed region (never inside it) the line also gets: the per-launch
p10 / p90, a cold-cache figure (each call after 512 MiB are written, so the
inputs are out of the 256 MiB last-level cache), the shader clock measured
while the forward runs back to back (``sclk_mhz_under_load``, from the
library's clock probe) with the matrix-core peak scaled to that clock
(``mfma_peak_at_measured_clock``), and for the 16-bit dense workloads the same
workload in the other 16-bit type (``companion``).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s + % of MI355X bf16 MFMA peak, B2 S4096 N24 D128"
PEAK_TFLOPS = {"bf16": 2500.0, "fp16": 2500.0, "fp32": 157.3}
HBM_GBPS = 8000.0
PEAK_CLOCK_MHZ = 2400.0  # the shader clock the published matrix-core peaks assume
COUNTERS = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
KERNEL_SOURCES = ["fa_mfma.hpp", "fa_mfma_pp.hpp", "fa_mfma_dispatch.hpp", "fa_device.hpp", "fa_params.h", "fa_mfma_bf16.hip",
                  "fa_mfma_f16.hip", "fa_generic.hip", "fa_launch.hip", "fa_merge.hip"]


# Default warm-up: the shader clock climbs for the first ~30 ms of back-to-back
# forward calls (B2 S4096 N24 D128 bf16: 389 -> 364 -> 355 -> 351 us per call
# over the first 100 calls, then flat at 350 for 500 more) and drops again
# after an idle second, so the timed steps start only after this much
# continuous work.
WARMUP_MS = 250
WARMUP_MIN = 20

# workloads whose element type --dtype chooses (the rest fix theirs)
DTYPE_WORKLOADS = ("c2_dense_bsnd", "c2_gqa_nkv4", "c2_mqa", "d256_dense_bsnd")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "attention_forward_fa_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps before the timed ones (default: as many as take %d ms, at least %d)"
                    % (WARMUP_MS, WARMUP_MIN))
    ap.add_argument("--workload", default="c2_dense_bsnd",
                    choices=["c2_dense_bsnd", "c3_causal", "c3_band", "c4_varlen_causal", "c5_varlen_sink_rope",
                             "c6_dense_pse", "c7_outer_split", "c2_gqa_nkv4", "c2_mqa", "d256_dense_bsnd"])
    ap.add_argument("--dtype", default="bf16", choices=["bf16", "fp16"])
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle CPU baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cold", action="store_true", help="skip the cold-cache figure")
    ap.add_argument("--no-clock", action="store_true", help="skip the shader-clock reading under load")
    ap.add_argument("--no-companion", action="store_true", help="skip the other 16-bit type's figure")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="launch one device copy of this many MiB (counter calibration runs)")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# FLOP and byte accounting
# ---------------------------------------------------------------------------

def kept_pairs(case, block: int = 0) -> int:
    """Kept (query, key) pairs; with block > 0, count whole block x block tiles that keep any pair."""
    import torch

    def seq_pairs(sq, skv):
        if sq == 0 or skv == 0:
            return 0
        band = case.atten_mask is not None or case.causal
        pre = case.pre_tokens if band else None
        nxt = (min(case.next_tokens, 0) if case.causal else case.next_tokens) if band else None
        if block == 0:
            i = torch.arange(sq, dtype=torch.int64)
            lo = torch.zeros_like(i) if pre is None else (i - pre).clamp(min=0)
            hi = torch.full_like(i, skv - 1) if nxt is None else (i + nxt).clamp(max=skv - 1)
            return int((hi - lo + 1).clamp(min=0).sum())
        total = 0
        for ib in range(0, sq, block):
            i0, i1 = ib, min(ib + block, sq) - 1
            lo = 0 if pre is None else max(0, i0 - pre)
            hi = skv - 1 if nxt is None else min(skv - 1, i1 + nxt)
            if hi < lo:
                continue
            jb0 = (lo // block) * block
            for jb in range(jb0, hi + 1, block):
                total += (i1 - i0 + 1) * (min(jb + block, skv) - jb)
        return total

    if case.layout == "TND":
        cu_q = case.cu_seqlens_q.tolist()
        cu_k = case.cu_seqlens_kv.tolist()
        per_head = sum(seq_pairs(cu_q[b + 1] - cu_q[b], cu_k[b + 1] - cu_k[b]) for b in range(len(cu_q) - 1))
        heads = case.q.shape[1]
        return per_head * heads
    B = case.q.shape[0]
    heads = case.q.shape[1] if case.layout == "BNSD" else case.q.shape[2]
    sq = case.q.shape[2] if case.layout == "BNSD" else case.q.shape[1]
    skv = case.k.shape[2] if case.layout == "BNSD" else case.k.shape[1]
    return seq_pairs(sq, skv) * B * heads


def flops_per_pair(case) -> int:
    d = case.q.shape[-1]
    dr = case.q_rope.shape[-1] if case.q_rope is not None else 0
    dv = case.v.shape[-1]
    return 2 * (d + dr) + 2 * dv


def algorithmic_bytes(case) -> int:
    """Inputs read once, output and statistics written once."""
    tot = 0
    for t in (case.q, case.k, case.v, case.q_rope, case.k_rope, case.atten_mask, case.sink, case.pse):
        if t is not None:
            tot += t.numel() * t.element_size()
    tot += case.q.numel() // case.q.shape[-1] * case.v.shape[-1] * case.q.element_size()  # O
    rows = case.q.numel() // case.q.shape[-1]
    tot += 2 * rows * 8 * 4  # softmax max / sum, 8 fp32 slots each
    return tot


def load_traffic(src_hash: str, workload: str, dtype: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on this kernel source (else None)."""
    if not os.path.exists(COUNTERS):
        return None
    with open(COUNTERS) as f:
        for line in f:
            parts = line.split()
            if not parts or parts[0].startswith("#") or len(parts) < 6:
                continue
            if parts[0] == workload and parts[1] == dtype and parts[2] == src_hash:
                return int(parts[5])
    return None


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample
# ---------------------------------------------------------------------------

def cpu_baseline(case, budget_s: float):
    import torch

    from oracle import attention as orc

    cores = len(os.sched_getaffinity(0))
    torch.set_num_threads(cores)
    B = case.q.shape[0] if case.layout != "TND" else 1
    heads = case.q.shape[2] if case.layout == "BSND" else case.q.shape[1]
    units, t0 = 0, time.perf_counter()
    fpp = flops_per_pair(case)
    if case.layout == "TND":
        cu = case.cu_seqlens_q.tolist()
        work = [(b, h) for b in range(len(cu) - 1) for h in range(heads)]
    else:
        work = [(b, h) for b in range(B) for h in range(heads)]
    # Walk the (sequence, head) units in order, wrapping round, until the time budget is spent.
    while True:
        b, h = work[units % len(work)]
        if case.layout == "TND":
            n = int(cu[b + 1] - cu[b])
        else:
            n = case.q.shape[1] if case.layout == "BSND" else case.q.shape[2]
        rows = torch.arange(n)
        orc.attention_forward(case.q, case.k, case.v, layout=case.layout, scale=case.scale, q_rope=case.q_rope,
                              k_rope=case.k_rope, atten_mask=case.atten_mask, sink=case.sink, causal=case.causal,
                              pre_tokens=case.pre_tokens, next_tokens=case.next_tokens,
                              cu_seqlens_q=case.cu_seqlens_q, cu_seqlens_kv=case.cu_seqlens_kv,
                              samples=[(b, h, rows)], pse=case.pse)
        units += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    total_pairs = kept_pairs(case, block=128)
    pairs = total_pairs * units / len(work)
    tflops = pairs * fpp / dt / 1e12
    cpu = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": round(tflops, 6), "unit": "TFLOP/s", "cores": torch.get_num_threads(), "kind": "oracle",
            "sample": f"{units} (sequence, head) units of the {len(work)} in the workload (wrapping round), every "
                      f"query row, float64, {dt:.1f} s; "
                      f"FLOPs scaled by the same 128x128 block accounting; CPU: {cpu}"}


# ---------------------------------------------------------------------------
# main
# ---------------------------------------------------------------------------

class Runner:
    """One workload resident on the GPU: its tensors, outputs, workspace and one step (phase 1 + phase 2)."""

    def __init__(self, case, workload, dev):
        import torch

        from attention_forward_fa_amd import _lib, api

        import synth

        self.case, self.torch, self._lib = case, torch, _lib
        g = {k: (v.to(dev) if v is not None else None) for k, v in case.tensors().items()}
        self.g = g
        self.nheads = case.q.shape[1] if case.layout in ("BNSD", "TND") else case.q.shape[2]
        self.out = torch.empty(case.q.shape[:-1] + (case.v.shape[-1],), dtype=case.q.dtype, device=dev)
        if case.layout == "TND":
            self.smax = torch.empty(self.nheads, case.q.shape[0], 8, dtype=torch.float32, device=dev)
        else:
            B = case.q.shape[0]
            S = case.q.shape[2] if case.layout == "BNSD" else case.q.shape[1]
            self.smax = torch.empty(B, self.nheads, S, 8, dtype=torch.float32, device=dev)
        self.ssum = torch.empty_like(self.smax)
        self.stream = torch.cuda.current_stream(dev)
        self.sh = self.stream.cuda_stream
        plan0 = api.ForwardPlan(g["q"], g["k"], g["v"], layout=case.layout, scale=case.scale, head_num=self.nheads,
                                query_rope=g["q_rope"], key_rope=g["k_rope"], atten_mask=g["atten_mask"],
                                sink=g["sink"], cu_seqlens_q=g["cu_seqlens_q"], cu_seqlens_kv=g["cu_seqlens_kv"],
                                causal=case.causal, pre_tokens=case.pre_tokens, next_tokens=case.next_tokens,
                                softmax_out_layout=case.softmax_out_layout, out=self.out, softmax_max=self.smax,
                                softmax_sum=self.ssum, real_shift=g["pse"])
        self.desc = plan0.describe()
        self.ws = plan0.workspace
        plan0.close()
        self.split = workload == "c7_outer_split"
        self.merge_ev = []
        if self.split:
            # the c2 problem as an outer split along the keys: one call per key chunk, then the merge
            cuts = synth.C7_CUTS
            self.chunks = []
            for a, b in zip(cuts[:-1], cuts[1:]):
                self.chunks.append((a, g["k"][:, a:b], g["v"][:, a:b], torch.empty_like(self.out),
                                    torch.empty_like(self.smax), torch.empty_like(self.ssum)))

    def step(self, ev_pair=None):
        case, g, _lib, sh, torch = self.case, self.g, self._lib, self.sh, self.torch
        if self.split:
            if ev_pair is not None:
                ev_pair[0].record(self.stream)
            for a, kc, vc, oc, mc, lc in self.chunks:
                wsz, h = _lib.fa_fwd_get_workspace_size(
                    g["q"], None, kc, None, vc, None, None, None, None, None, None, a, case.scale, 1.0,
                    case.pre_tokens, case.next_tokens, self.nheads, case.layout, 0, 0, case.causal, "", mc, lc, oc)
                _lib.fa_fwd(None, wsz, h, sh)
                _lib.fa_plan_destroy(h)
            if ev_pair is not None:
                ev_pair[1].record(self.stream)
                em = torch.cuda.Event(enable_timing=True)
                em.record(self.stream)
            _lib.fa_fwd_merge([c[3] for c in self.chunks], [c[4] for c in self.chunks], [c[5] for c in self.chunks],
                              case.layout, self.nheads, "", self.out, self.smax, self.ssum, sh)
            if ev_pair is not None:
                em2 = torch.cuda.Event(enable_timing=True)
                em2.record(self.stream)
                self.merge_ev.append((em, em2))
            return
        # phase 1 + phase 2; the workspace is allocated once, outside the timed region
        wsz, h = _lib.fa_fwd_get_workspace_size(
            g["q"], g["q_rope"], g["k"], g["k_rope"], g["v"], g["pse"], g["atten_mask"], g["sink"], g["cu_seqlens_q"],
            g["cu_seqlens_kv"], None, None, case.scale, 1.0, case.pre_tokens, case.next_tokens, self.nheads,
            case.layout, 0, 0, case.causal, case.softmax_out_layout, self.smax, self.ssum, self.out)
        if ev_pair is not None:
            ev_pair[0].record(self.stream)
        _lib.fa_fwd(self.ws, wsz, h, sh)
        if ev_pair is not None:
            ev_pair[1].record(self.stream)
        _lib.fa_plan_destroy(h)

    def timed(self, steps, warmup):
        """W untimed steps (None: at least WARMUP_MIN, until WARMUP_MS of them have run), then K steps
        between two synchronisations: (wall seconds, per-launch ms list, warm-up steps run)."""
        torch = self.torch
        done = 0
        t_w = time.perf_counter()
        while (done < warmup) if warmup is not None else (
                done < WARMUP_MIN or (time.perf_counter() - t_w) * 1e3 < WARMUP_MS):
            self.step()
            done += 1
            if warmup is None and done % 10 == 0:
                torch.cuda.synchronize()  # wall time then follows the GPU
        torch.cuda.synchronize()
        events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            self.step(events[i])
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        return elapsed, [a.elapsed_time(b) for a, b in events], done

    def cold(self, n, dev):
        """Per-launch ms with the caches flushed first: 512 MiB written before each call (the last-level
        cache holds 256 MiB), one call at a time."""
        torch = self.torch
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        out = []
        for _ in range(n):
            flush.fill_(1)
            ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            self.step(ev)
            torch.cuda.synchronize()
            out.append(ev[0].elapsed_time(ev[1]))
        del flush
        return out

    def clock_under_load(self, dev, window_us=150000):
        """Shader clock while the forward runs back to back: the library's clock probe idles on a side
        stream (default priority) for window_us while this stream keeps launching steps."""
        torch, _lib = self.torch, self._lib
        probe = torch.zeros(2, dtype=torch.int64, device=dev)
        side = torch.cuda.Stream(device=dev)
        for _ in range(3):
            self.step()
        torch.cuda.synchronize()
        _lib.fa_clock_probe(window_us, probe, side.cuda_stream)
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < window_us * 1.2e-6:
            self.step()
        torch.cuda.synchronize()
        cycles, ticks = (int(x) for x in probe.cpu().tolist())
        return cycles / (ticks / 100e6) / 1e6 if ticks > 0 else None


def pct(xs, q):
    ys = sorted(xs)
    return ys[min(len(ys) - 1, max(0, int(round(q / 100.0 * (len(ys) - 1)))))]


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(head / batch sharding needs no collective; see the design notes).", file=sys.stderr)
        sys.exit(2)

    import torch

    import synth

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    dtype_choice = args.workload in DTYPE_WORKLOADS
    case = synth.workload(args.workload, args.dtype) if dtype_choice else synth.workload(args.workload)
    dtype = {torch.bfloat16: "bf16", torch.float16: "fp16", torch.float32: "fp32"}[case.q.dtype]

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        print(f"[bench] copy calibration: {args.copy_calibration_mib} MiB read + written", file=sys.stderr)
        del a, b

    run = Runner(case, args.workload, dev)
    desc = run.desc
    elapsed, kernel_ms, warmup_done = run.timed(args.steps, args.warmup)
    kernel_ms_avg = sum(kernel_ms) / len(kernel_ms)
    kernel_ms_med = pct(kernel_ms, 50)

    pairs_blk = kept_pairs(case, block=128)
    pairs_exact = kept_pairs(case, block=0)
    fpp = flops_per_pair(case)
    flops = pairs_blk * fpp
    ms_per_step = elapsed * 1e3 / args.steps
    value = flops / (ms_per_step * 1e-3) / 1e12
    peak = PEAK_TFLOPS[dtype]
    src_hash = kernel_source_hash()
    traffic = load_traffic(src_hash, args.workload, dtype)
    abytes = algorithmic_bytes(case)
    tf = lambda ms: round(flops / (ms * 1e-3) / 1e12, 2)
    # The dominant kernel's roofline: matrix-core bound when the workload's arithmetic intensity
    # (FLOP per algorithmic byte) is above the ridge point peak / HBM bandwidth, else HBM bound.
    if flops / abytes >= peak * 1e12 / (HBM_GBPS * 1e9):
        roof = {"bound": "mfma", "achieved": tf(kernel_ms_avg), "peak": peak, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(abytes / (kernel_ms_avg * 1e-3) / 1e9, 1), "peak": HBM_GBPS,
                "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = traffic
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": warmup_done,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic: iid N(0,1) q/k/v drawn in fp32 from a fixed seed, rounded to the dtype",
        "config": {"workload": args.workload, "layout": case.layout, "q_shape": list(case.q.shape),
                   "kv_heads": case.k.shape[1] if case.layout in ("BNSD", "TND") else case.k.shape[2],
                   "causal": case.causal, "mask": case.atten_mask is not None,
                   "pre_tokens": case.pre_tokens, "next_tokens": case.next_tokens,
                   "rope_dim": case.q_rope.shape[-1] if case.q_rope is not None else 0,
                   "sink": case.sink is not None, "pse": case.pse is not None, "scale": case.scale},
        "pct_of_mfma_peak": round(100.0 * value / peak, 2),
        "roofline": roof,
        "kernel": {"name": "fa_fwd_" + desc.split()[0].split("=")[1], "plan": desc,
                   "avg_ms": round(kernel_ms_avg, 5), "median_ms": round(kernel_ms_med, 5),
                   "p10_ms": round(pct(kernel_ms, 10), 5), "p90_ms": round(pct(kernel_ms, 90), 5),
                   "flops_per_launch": flops, "flops_exact_pairs": pairs_exact * fpp,
                   "algorithmic_bytes_per_launch": abytes,
                   "achieved_TFLOPs": tf(kernel_ms_avg),
                   "achieved_GBps_algorithmic": round(abytes / (kernel_ms_avg * 1e-3) / 1e9, 1),
                   "source_hash": src_hash},
    }
    if run.split:
        n_o = run.out.numel() * run.out.element_size()
        n_st = run.smax.numel() * 4
        merge_bytes = len(run.chunks) * (n_o + 2 * n_st) + n_o + 2 * n_st
        merge_ms = sum(a.elapsed_time(b) for a, b in run.merge_ev) / len(run.merge_ev)
        result["config"]["key_chunks"] = list(synth.C7_CUTS)
        result["merge_kernel"] = {"avg_ms": round(merge_ms, 5), "bytes_per_launch": merge_bytes,
                                  "achieved_GBps": round(merge_bytes / (merge_ms * 1e-3) / 1e9, 1),
                                  "frac_of_hbm": round(merge_bytes / (merge_ms * 1e-3) / 1e9 / HBM_GBPS, 4)}
        result["kernel"]["note"] = "avg_ms covers the forward calls of all key chunks; the merge is timed apart"
    if not args.no_cold:
        cold = run.cold(max(5, args.steps // 4), dev)
        cold_ms = pct(cold, 50)
        result["kernel"]["cold_median_ms"] = round(cold_ms, 5)
        result["kernel"]["cold_tflops"] = tf(cold_ms)
        result["kernel"]["cold_note"] = "one call at a time after writing 512 MiB (the inputs leave the 256 MiB " \
                                        "last-level cache); the timed steps above run back to back on warm caches"
    if not args.no_clock:
        mhz = run.clock_under_load(dev)
        result["sclk_mhz_under_load"] = round(mhz, 1) if mhz else None
        if mhz and roof["bound"] == "mfma":
            # the matrix-core peak scaled to the clock the chip held while the forward ran (the published
            # peak assumes PEAK_CLOCK_MHZ): how much of the matrix-core time the kernel keeps busy, apart
            # from the box's clock; roofline.frac above stays against the published peak
            p_clk = peak * mhz / PEAK_CLOCK_MHZ
            result["mfma_peak_at_measured_clock"] = {"sclk_mhz": round(mhz, 1), "peak": round(p_clk, 1),
                                                     "unit": "TFLOP/s", "frac": round(roof["achieved"] / p_clk, 4)}
    if args.workload in DTYPE_WORKLOADS and not args.no_companion:
        # the same workload in the other 16-bit type, timed the same way
        other = "fp16" if dtype == "bf16" else "bf16"
        del run
        torch.cuda.empty_cache()
        run2 = Runner(synth.workload(args.workload, other), args.workload, dev)
        el2, ms2, _ = run2.timed(args.steps, args.warmup)
        avg2 = sum(ms2) / len(ms2)
        result["companion"] = {"dtype": other, "value": round(flops / (el2 / args.steps) / 1e12, 2),
                               "kernel_avg_ms": round(avg2, 5), "kernel_median_ms": round(pct(ms2, 50), 5),
                               "achieved_TFLOPs": tf(avg2), "frac": round(tf(avg2) / PEAK_TFLOPS[other], 4),
                               "plan": run2.desc}
        del run2
    print(f"[bench] {args.workload} {dtype}: {value:.1f} TFLOP/s, kernel {kernel_ms_avg:.4f} ms avg", file=sys.stderr,
          flush=True)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
