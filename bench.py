#!/usr/bin/env python3
"""Benchmark of the fused attention forward hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
the prefill kernel on the dense MHA causal workload the pages' forward TFLOPS
table is quoted on (b=1, h=16, s_q=s_k=8192, d=128, bottom-right causal,
O + LSE), then the split-KV decode of the MQA decode workload (B=64
sequences, one query token, h_q=128, h_kv=1, KV lengths uniform in
[1024, 8192], chunks of 512, then the LSE merge) at d=128 and at d=256.
Inputs are resident in HBM before the timed region, and each case rotates
over at least 3 input sets that together hold more than twice the 256 MB
last-level cache, so repeated steps do not read their inputs out of it.

`value` is the prefill throughput in TFLOP/s counted as 4*d per visible
(query, key) pair (causal-adjusted); the decode throughputs in GB/s
(algorithmic bytes: K and V of every cached token plus Q, O and LSE) are
reported beside it.  Before the warm-up steps a settle pass runs the prefill
back to back until the clock has settled (settle()), so that a short warm-up
does not time the clock ramp of a cold GPU.  Kernel times come from HIP events
recorded on the stream the kernels run on: the K timed steps run as K prefill
launches, then K decode passes at each head dim, each block between two
events (see timed()).  A separate pass afterwards brackets each of up to 100
further launches with events of its own and reports the median, p10 and p90
of single launches beside the block average (launch_spread()), and a last
pass of about one second of back-to-back prefill launches reads the GFX clock
through amdsmi, so that the prefill fraction is also given against the bf16
peak at the clock the chip ran at (sampled_clock(), clock_fraction()).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME | --all]
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # 256 CUs x 2.4 GHz x 4096 dense bf16 flop/clk/CU
PEAK_HBM_GBS = 8000.0
HEADLINE_PREFILL = "mha_b1_h16_s8192_d128_causal"
HEADLINE_DECODE = "mqa_decode_B64_hq128_d128"
SECOND_DECODE = "mqa_decode_B64_hq128_d256"
MALL_BYTES = 256 << 20  # last-level (Infinity) cache of the MI355X


def visible_pairs(s_q: int, s_k: int, causal: bool, window: int) -> int:
    """Number of (query row, key) pairs the mask keeps (closed form per row)."""
    off = s_k - s_q
    total = 0
    for i in range(s_q):
        hi = s_k - 1 if not causal else min(s_k - 1, i + off)
        lo = 0 if window <= 0 else max(0, i + off - window + 1)
        if hi >= lo:
            total += hi - lo + 1
    return total


def prefill_flops(w) -> int:
    return 4 * w.d * w.b * w.h_q * visible_pairs(w.s_q, w.s_k, w.causal, w.window)


def decode_bytes(w, total_tokens: int) -> int:
    kv = total_tokens * w.h_kv * w.d * 2 * (1 if w.fp8 else 2)  # K and V, 1 byte per FP8 code
    qo = 2 * w.b * w.h_q * w.d * 2
    return kv + qo + w.b * w.h_q * 4


def n_sets_beyond_mall(bytes_per_set: int) -> int:
    """Input sets to rotate over so that repeated steps cannot be served from the MALL.

    At least 3 independent sets, and together more than twice the 256 MB
    last-level cache: a launch then never finds its inputs left in that cache
    by the launch before it.  At most 32 sets: only the tiny single-head
    workload (latency, not bandwidth) would ask for more.
    """
    return min(32, max(3, -(-2 * MALL_BYTES // max(1, bytes_per_set))))


def prefill_set_bytes(w) -> int:
    return 2 * w.b * w.d * (w.h_q * w.s_q + 2 * w.h_kv * w.s_k)


def decode_set_bytes(w) -> int:
    tokens = w.b * (w.len_lo + w.len_hi) // 2  # expected cache size of the draw
    return tokens * w.h_kv * w.d * 2 * (1 if w.fp8 else 2) + w.b * w.h_q * w.d * 2


class PrefillCase:
    def __init__(self, w, n_sets: int, dev):
        import torch

        from attention_forward_attn_amd.inputs import prefill_inputs

        self.w = w
        self.scale = 1.0 / math.sqrt(w.d)
        inp = prefill_inputs(w.b, w.h_q, w.h_kv, w.s_q, w.s_k, w.d, w.seed, w.sinks)
        self.sets = [{k: (v.to(dev) if v is not None else None) for k, v in inp.items()}]
        gen = torch.Generator(device=dev).manual_seed(w.seed + 1)
        for _ in range(1, n_sets):  # more sets of the same shapes, drawn on the device
            st = {n: torch.randn(self.sets[0][n].shape, generator=gen, device=dev).to(torch.bfloat16)
                  for n in ("q", "k", "v")}
            st["sinks"] = self.sets[0]["sinks"]
            self.sets.append(st)
        self.out = torch.empty((w.b, w.h_q, w.s_q, w.d), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((w.b, w.h_q, w.s_q), dtype=torch.float32, device=dev)
        self.flops = prefill_flops(w)
        # workspace of the chunked schedule (d = 512 causal), allocated once outside the timed loop
        import ctypes

        import attention_forward_attn_amd as afa

        s0 = self.sets[0]
        a = afa._binding.prefill_args(s0["q"], s0["k"], s0["v"], self.out, self.lse, s0["sinks"], self.scale,
                                      w.causal, w.window)
        need = int(afa.load_library().attn_fwd_prefill_chunked_workspace_size(ctypes.byref(a)))
        self.workspace = torch.zeros(need, dtype=torch.uint8, device=dev) if need else None  # zeroed queue header

    def run(self, i: int):
        import attention_forward_attn_amd as afa

        s = self.sets[i % len(self.sets)]
        afa.prefill(s["q"], s["k"], s["v"], scale=self.scale, causal=self.w.causal,
                    window=self.w.window, sinks=s["sinks"], out=self.out, lse=self.lse,
                    workspace=self.workspace)


class DecodeCase:
    def __init__(self, w, n_sets: int, dev):
        import torch

        import attention_forward_attn_amd as afa
        from attention_forward_attn_amd.inputs import decode_inputs

        self.w = w
        base = decode_inputs(w.b, w.h_q, w.h_kv, w.d, w.len_lo, w.len_hi, w.seed, w.sinks)
        self.total = int(base["kv_len"].sum())
        self.max_len = int(base["kv_len"].max())
        self.kv_start = base["kv_start"].to(dev)
        self.kv_len = base["kv_len"].to(dev)
        self.sets = [{"q": base["q"].to(dev), "k": base["k"].to(dev), "v": base["v"].to(dev)}]
        gen = torch.Generator(device=dev).manual_seed(w.seed + 1)
        for _ in range(1, n_sets):  # more sets of the same shapes, drawn on the device
            self.sets.append({n: torch.randn(t.shape, generator=gen, device=dev).to(torch.bfloat16)
                              for n, t in self.sets[0].items()})
        self.sinks = base["sinks"].to(dev) if base["sinks"] is not None else None
        self.scale = 1.0 / math.sqrt(w.d)
        self.ws = afa.new_decode_workspace(afa.decode_workspace_size(w.b, w.h_q, w.d, self.max_len, w.split),
                                           dev)
        self.out = torch.empty((w.b, w.h_q, w.d), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((w.b, w.h_q), dtype=torch.float32, device=dev)
        self.bytes = decode_bytes(w, self.total)

    def run(self, i: int):
        import attention_forward_attn_amd as afa

        s = self.sets[i % len(self.sets)]
        afa.decode(s["q"], s["k"], s["v"], self.kv_start, self.kv_len, self.max_len,
                   scale=self.scale, sinks=self.sinks, split_size=self.w.split, workspace=self.ws,
                   out=self.out, lse=self.lse)


def cpu_baseline_prefill(w, budget_s: float = 12.0):
    """Time the fp64 oracle on whole heads of the same workload until the budget is spent."""
    import numpy as np
    import torch

    import oracle
    from attention_forward_attn_amd.inputs import prefill_inputs

    try:
        from threadpoolctl import threadpool_info

        cores = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] + [1])
    except Exception:  # pragma: no cover - threadpoolctl is optional
        cores = os.cpu_count() or 1
    inp = prefill_inputs(w.b, w.h_q, w.h_kv, w.s_q, w.s_k, w.d, w.seed, w.sinks)
    q = inp["q"].to(torch.float64).numpy()
    k = inp["k"].to(torch.float64).numpy()
    v = inp["v"].to(torch.float64).numpy()
    sig = inp["sinks"].to(torch.float64).numpy() if inp["sinks"] is not None else None
    ratio = w.h_q // w.h_kv
    done = 0
    t0 = time.perf_counter()
    for bi in range(w.b):
        for h in range(w.h_q):
            g = h // ratio
            oracle.attention_ref(q[bi:bi + 1, h:h + 1], k[bi:bi + 1, g:g + 1], v[bi:bi + 1, g:g + 1],
                                 1.0 / math.sqrt(w.d), causal=w.causal, window=w.window,
                                 sinks=None if sig is None else sig[h:h + 1])
            done += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    flops = 4 * w.d * done * visible_pairs(w.s_q, w.s_k, w.causal, w.window)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{done} of {w.b * w.h_q} (batch, head) slices of {w.name}, fp64 numpy, "
                      f"{dt:.1f} s",
            "threads": f"matrix products on {cores} BLAS threads, elementwise steps on one thread",
            "cpu_model": cpu_model(), "host_cpus": len(os.sched_getaffinity(0))}


def cpu_model() -> str:
    """The host CPU's model name (first `model name` line of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


def timed(cases, steps: int, warmup: int, start: int = 0):
    """Run warmup + steps; return (per-case mean ms per launch, wall ms per step).

    The W warm-up steps run case by case, last case first; the timed region
    then runs the K steps case by case: K launches of the first case back to
    back, then K of the next, each block between two HIP events on the launch
    stream (torch's current stream), so a per-launch average carries no event
    overhead of its own.  Every launch takes the next input
    set of its case's rotation, as a step would.  The region is bracketed by
    torch.cuda.synchronize() on both sides.
    """
    import torch

    # warm-up in blocks, last case first, so that each timed block follows warm
    # launches of its own kind (a memory-bound decode block leaves the clock
    # in another state than a compute-bound prefill block)
    for c in reversed(cases):
        for i in range(warmup):
            c.run(start + i)
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(cases) + 1)]
    t0 = time.perf_counter()
    evs[0].record()
    for j, c in enumerate(cases):
        for i in range(steps):
            c.run(start + warmup + i)
        evs[j + 1].record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    per = [evs[j].elapsed_time(evs[j + 1]) / steps for j in range(len(cases))]
    return per, wall_ms


def settle(case, start: int, min_s: float = 1.0, max_s: float = 8.0, block: int = 10, tol: float = 0.02):
    """Run the case back to back until the GPU clock has settled; returns what it took.

    A pass of its own before the warm-up steps, so that the timed steps do not
    fall into the clock ramp of a cold GPU (a fresh box needs on the order of
    a few hundred launches of this kind before its launch time stops
    falling).  Launches go in blocks of `block`, each block between two
    events; the pass ends once at least `min_s` seconds have passed and the
    last two block averages agree within `tol`, or after `max_s` seconds.
    """
    import torch

    t0 = time.perf_counter()
    blocks, i = [], start
    while True:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(block):
            case.run(i)
            i += 1
        b.record()
        b.synchronize()
        blocks.append(a.elapsed_time(b) / block)
        el = time.perf_counter() - t0
        steady = len(blocks) >= 2 and abs(blocks[-1] - blocks[-2]) <= tol * blocks[-2]
        if (el >= min_s and steady) or el >= max_s:
            break
    return {"seconds": round(time.perf_counter() - t0, 2), "launches": i - start, "steady": steady,
            "first_block_ms": round(blocks[0], 4), "last_blocks_ms": [round(x, 4) for x in blocks[-2:]]}


def launch_spread(case, n: int, start: int):
    """Per-launch times (ms) of n launches, each between two events of its own.

    Run after the timed block, outside it: events around every launch keep the
    launches from running back to back, so these figures describe the spread
    of single launches (median, p10, p90), while the block average is the
    throughput.
    """
    import torch

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i, (a, b) in enumerate(evs):
        a.record()
        case.run(start + i)
        b.record()
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in evs)
    pick = lambda q: t[min(n - 1, int(round(q * (n - 1))))]
    return {"launches": n, "median_ms": round(pick(0.5), 4), "p10_ms": round(pick(0.1), 4),
            "p90_ms": round(pick(0.9), 4)}


def _smi_handle(dev_index: int):
    """amdsmi handle of torch device dev_index, matched by PCI domain and bus."""
    import amdsmi
    import torch

    props = torch.cuda.get_device_properties(dev_index)
    handles = amdsmi.amdsmi_get_processor_handles()
    for hd in handles:
        bdf = amdsmi.amdsmi_get_gpu_device_bdf(hd)  # "dddd:bb:dd.f"
        dom, bus = bdf.split(":")[:2]
        if int(dom, 16) == props.pci_domain_id and int(bus, 16) == props.pci_bus_id:
            return hd
    return handles[0] if len(handles) == 1 else None


CLOCK_MHZ_RANGE = (500, 2600)  # plausible GFX clocks of a loaded MI355X (2400 MHz peak)


def pick_clock(metrics_mhz, info_mhz):
    """Choose the clock reading to price the peak at, or explain why there is none.

    metrics_mhz: per-XCD medians of amdsmi's GPU-metrics `current_gfxclks`;
    info_mhz: median of amdsmi_get_clock_info(GFX)["clk"].  A source is used
    only if its reading lies in CLOCK_MHZ_RANGE; the per-XCD metrics come
    first, the clock-info reading second.  Returns (mhz, source) or
    (None, reason).
    """
    lo, hi = CLOCK_MHZ_RANGE
    if metrics_mhz:
        mhz = sorted(metrics_mhz)[len(metrics_mhz) // 2]
        if lo <= mhz <= hi:
            return mhz, "gpu_metrics.current_gfxclks"
    if info_mhz is not None and lo <= info_mhz <= hi:
        return info_mhz, "clock_info.gfx"
    return None, (f"no plausible clock reading (per-XCD metrics {metrics_mhz}, clock info {info_mhz} MHz; "
                  f"expected {lo}-{hi} MHz)")


def clock_fraction(clock: dict, achieved: float) -> dict:
    """Add peak_at_clock / frac_at_clock to a sampled_clock() result, or an error entry.

    A fraction above 1 cannot happen on a correct clock reading (the peak is
    linear in the clock), so it is reported as an error instead.
    """
    out = dict(clock)
    mhz = out.get("gfx_mhz")
    if mhz is None:
        out.setdefault("error", "no clock reading")
        return out
    peak = PEAK_BF16_TFLOPS * mhz / 2400.0
    frac = achieved / peak
    if frac > 1.0:
        out["error"] = (f"{achieved:.1f} TFLOP/s exceeds the peak at the sampled {mhz} MHz "
                        f"({peak:.1f} TFLOP/s): the clock reading is wrong")
        return out
    out["peak_at_clock"] = round(peak, 1)
    out["frac_at_clock"] = round(frac, 4)
    return out


def sampled_clock(case, start: int, ms_per_launch: float, seconds: float = 1.0):
    """GFX clock while the case runs back to back, read through amdsmi.

    A pass of its own after the timed block: about `seconds` of back-to-back
    launches while a thread reads the device's clock every 10 ms from two
    amdsmi sources: the GPU metrics table (per XCD, where it lists them) and
    the GFX clock info.  Samples from the second half of the pass (steady
    clock) are kept; the medians are reported raw, and pick_clock() chooses
    the one that is plausible.  The bf16 dense peak is linear in the clock
    (4096 flop per CU and cycle), so the peak at the sampled clock is
    2516.6 x clk / 2400 TFLOP/s (clock_fraction()).  Returns {"error": ...}
    when amdsmi cannot read the clock; the timed figures do not depend on this
    pass.
    """
    import threading

    import torch

    try:
        import amdsmi

        amdsmi.amdsmi_init()
    except Exception as e:  # no amdsmi or no driver access
        return {"error": f"amdsmi unavailable: {e}"}
    try:
        hd = _smi_handle(torch.cuda.current_device())
        if hd is None:
            return {"error": "no amdsmi device matches the torch device"}

        def read():
            xs, ci = [], None
            try:
                clks = amdsmi.amdsmi_get_gpu_metrics_info(hd).get("current_gfxclks")
                if isinstance(clks, list):
                    xs = [c for c in clks if isinstance(c, int) and 0 < c < 10000]
            except Exception:
                pass
            try:
                c = amdsmi.amdsmi_get_clock_info(hd, amdsmi.AmdSmiClkType.GFX).get("clk")
                ci = c if isinstance(c, int) and c > 0 else None
            except Exception:
                pass
            return xs, ci

        samples, stop = [], threading.Event()

        def sampler():
            while not stop.is_set():
                samples.append((time.perf_counter(), read()))
                stop.wait(0.01)

        n = max(100, int(seconds / (ms_per_launch * 1e-3)))
        th = threading.Thread(target=sampler, daemon=True)
        t0 = time.perf_counter()
        th.start()
        for i in range(n):
            case.run(start + i)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        stop.set()
        th.join()
        kept = [r for t, r in samples if t >= t0 + 0.5 * (t1 - t0)]
        if not kept:
            return {"error": "no clock samples while the kernels ran"}
        mets = [xs for xs, _ in kept if xs]
        per_xcd = ([sorted(col)[len(col) // 2] for col in zip(*mets)]
                   if mets and len({len(x) for x in mets}) == 1 else [])
        infos = sorted(ci for _, ci in kept if ci is not None)
        info = infos[len(infos) // 2] if infos else None
        mhz, src = pick_clock(per_xcd, info)
        out = {"launches": n, "samples": len(kept), "metrics_mhz_per_xcd": per_xcd, "clock_info_mhz": info}
        if mhz is None:
            out["error"] = src
        else:
            out["gfx_mhz"] = mhz
            out["source"] = src
        return out
    except Exception as e:
        return {"error": f"clock sampling failed: {e}"}
    finally:
        try:
            amdsmi.amdsmi_shut_down()
        except Exception:
            pass


def kernel_source_hash(unit: str) -> str:
    """Short hash of one HIP translation unit and every source it includes.

    A recorded counter profile is valid only for the hash of the unit that
    holds its kernel: a change anywhere in that unit's include closure voids it.
    """
    import hashlib
    import re

    d = os.path.join(ROOT, "attention_forward_attn_amd", "csrc")
    seen, todo = set(), [unit]
    while todo:
        f = todo.pop()
        if f in seen:
            continue
        seen.add(f)
        with open(os.path.join(d, f)) as fh:
            todo += [m for m in re.findall(r'^#include "([^"/]+)"', fh.read(), re.M)]
    h = hashlib.sha256()
    for f in sorted(seen):
        h.update(f.encode())
        with open(os.path.join(d, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(*profiles: str):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, calibrated) from committed profile summaries.

    Each summary ends with a `traffic_record:` line naming the translation unit
    of its kernel and that unit's source hash when it was measured.  Returns
    (bytes, note): the bytes are None if any summary is missing or was taken
    on other sources.  The counters are not read in the bench run itself; the
    note says where the figure was recorded.
    """
    total = 0
    for name in profiles:
        path = os.path.join(ROOT, "profiles", name)
        if not os.path.exists(path):
            return None, f"no recorded counters (profiles/{name} missing)"
        rec = None
        with open(path) as fh:
            for line in fh:
                if line.startswith("traffic_record:"):
                    rec = dict(kv.split("=", 1) for kv in line.split()[1:])
        if rec is None or "src" not in rec:
            return None, f"profiles/{name} has no traffic record"
        if rec.get("kernel_src_sha") != kernel_source_hash(rec["src"]):
            return None, f"profiles/{name} was taken on other sources of {rec['src']}"
        total += int(float(rec["fetch_bytes"])) + int(float(rec["write_bytes"]))
    return total, ("recorded, not counted in this run: FETCH_SIZE + WRITE_SIZE per launch from "
                   + ", ".join(f"profiles/{n}" for n in profiles) + " (current kernel sources)")


PREFILL_PROFILE = ("prefill_d128_mha_b1_h16_s8192_d128_causal.md",)
DECODE_PROFILES = {"mqa_decode_B64_hq128_d128": ("decode_d128_mqa_decode_B64_hq128_d128.md",),
                   "mqa_decode_B64_hq128_d256": ("decode_d256_mqa_decode_B64_hq128_d256.md",)}


def roofline_prefill(flops: int, ms: float, traffic=(None, None)):
    achieved = flops / (ms * 1e-3) / 1e12
    r = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
         "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic[0]}
    if traffic[1]:
        r["traffic_source"] = traffic[1]
    return r


def roofline_decode(nbytes: int, ms: float, traffic=(None, None)):
    achieved = nbytes / (ms * 1e-3) / 1e9
    r = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
         "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic[0]}
    if traffic[1]:
        r["traffic_source"] = traffic[1]
    return r


class PagedDecodeCase(DecodeCase):
    """The decode workload held in a paged cache (block table of page_size-token pages)."""

    def __init__(self, w, n_sets: int, dev):
        import torch

        import attention_forward_attn_amd as afa
        from attention_forward_attn_amd.inputs import paged_decode_inputs

        self.w = w
        base = paged_decode_inputs(w.b, w.h_q, w.h_kv, w.d, w.len_lo, w.len_hi, w.page_size, w.seed, w.sinks)
        self.total = int(base["kv_len"].sum())
        self.max_len = int(base["kv_len"].max())
        self.kv_len = base["kv_len"].to(dev)
        self.table = base["block_table"].to(dev)
        self.sets = [{"q": base["q"].to(dev), "k": base["k_cache"].to(dev), "v": base["v_cache"].to(dev)}]
        gen = torch.Generator(device=dev).manual_seed(w.seed + 1)
        for _ in range(1, n_sets):
            self.sets.append({n: torch.randn(t.shape, generator=gen, device=dev).to(torch.bfloat16)
                              for n, t in self.sets[0].items()})
        self.sinks = base["sinks"].to(dev) if base["sinks"] is not None else None
        self.scale = 1.0 / math.sqrt(w.d)
        self.ws = afa.new_decode_workspace(afa.decode_workspace_size(w.b, w.h_q, w.d, self.max_len, w.split),
                                           dev)
        self.out = torch.empty((w.b, w.h_q, w.d), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((w.b, w.h_q), dtype=torch.float32, device=dev)
        self.bytes = decode_bytes(w, self.total)

    def run(self, i: int):
        import attention_forward_attn_amd as afa

        s = self.sets[i % len(self.sets)]
        afa.decode_paged(s["q"], s["k"], s["v"], self.table, self.kv_len, self.max_len,
                         scale=self.scale, sinks=self.sinks, split_size=self.w.split, workspace=self.ws,
                         out=self.out, lse=self.lse)


class Fp8DecodeCase(DecodeCase):
    """The decode workload with K and V as E4M3 codes and per-kv-head scales."""

    def __init__(self, w, n_sets: int, dev):
        import torch

        import attention_forward_attn_amd as afa
        from attention_forward_attn_amd.inputs import fp8_decode_inputs

        self.w = w
        base = fp8_decode_inputs(w.b, w.h_q, w.h_kv, w.d, w.len_lo, w.len_hi, w.seed, w.sinks)
        self.total = int(base["kv_len"].sum())
        self.max_len = int(base["kv_len"].max())
        self.kv_start = base["kv_start"].to(dev)
        self.kv_len = base["kv_len"].to(dev)
        self.k_scale = base["k_scale"].to(dev)
        self.v_scale = base["v_scale"].to(dev)
        self.sets = [{"q": base["q"].to(dev), "k": base["k8"].to(dev), "v": base["v8"].to(dev)}]
        gen = torch.Generator(device=dev).manual_seed(w.seed + 1)
        for _ in range(1, n_sets):  # further sets: fresh codes of the same shapes (no NaN codes)
            st = {"q": torch.randn(self.sets[0]["q"].shape, generator=gen, device=dev).to(torch.bfloat16)}
            for n in ("k", "v"):
                st[n] = torch.randint(0, 0x7f, self.sets[0][n].shape, generator=gen, device=dev,
                                      dtype=torch.int32).to(torch.uint8) | (
                    torch.randint(0, 2, self.sets[0][n].shape, generator=gen, device=dev,
                                  dtype=torch.int32).to(torch.uint8) << 7)
            self.sets.append(st)
        self.sinks = base["sinks"].to(dev) if base["sinks"] is not None else None
        self.scale = 1.0 / math.sqrt(w.d)
        self.ws = afa.new_decode_workspace(afa.decode_workspace_size(w.b, w.h_q, w.d, self.max_len, w.split),
                                           dev)
        self.out = torch.empty((w.b, w.h_q, w.d), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((w.b, w.h_q), dtype=torch.float32, device=dev)
        self.bytes = decode_bytes(w, self.total)

    def run(self, i: int):
        import attention_forward_attn_amd as afa

        s = self.sets[i % len(self.sets)]
        afa.decode_fp8(s["q"], s["k"], s["v"], self.k_scale, self.v_scale, self.kv_start, self.kv_len,
                       self.max_len, scale=self.scale, sinks=self.sinks, split_size=self.w.split,
                       workspace=self.ws, out=self.out, lse=self.lse)


class PagedFp8DecodeCase(DecodeCase):
    """The FP8 decode workload held in a paged cache (block table of page_size-token pages)."""

    def __init__(self, w, n_sets: int, dev):
        import torch

        import attention_forward_attn_amd as afa
        from attention_forward_attn_amd.inputs import paged_fp8_decode_inputs

        self.w = w
        base = paged_fp8_decode_inputs(w.b, w.h_q, w.h_kv, w.d, w.len_lo, w.len_hi, w.page_size, w.seed, w.sinks)
        self.total = int(base["kv_len"].sum())
        self.max_len = int(base["kv_len"].max())
        self.kv_len = base["kv_len"].to(dev)
        self.table = base["block_table"].to(dev)
        self.k_scale = base["k_scale"].to(dev)
        self.v_scale = base["v_scale"].to(dev)
        self.sets = [{"q": base["q"].to(dev), "k": base["k8_cache"].to(dev), "v": base["v8_cache"].to(dev)}]
        gen = torch.Generator(device=dev).manual_seed(w.seed + 1)
        for _ in range(1, n_sets):  # further sets: fresh codes of the same shapes (no NaN codes)
            st = {"q": torch.randn(self.sets[0]["q"].shape, generator=gen, device=dev).to(torch.bfloat16)}
            for n in ("k", "v"):
                st[n] = torch.randint(0, 0x7f, self.sets[0][n].shape, generator=gen, device=dev,
                                      dtype=torch.int32).to(torch.uint8) | (
                    torch.randint(0, 2, self.sets[0][n].shape, generator=gen, device=dev,
                                  dtype=torch.int32).to(torch.uint8) << 7)
            self.sets.append(st)
        self.sinks = base["sinks"].to(dev) if base["sinks"] is not None else None
        self.scale = 1.0 / math.sqrt(w.d)
        self.ws = afa.new_decode_workspace(afa.decode_workspace_size(w.b, w.h_q, w.d, self.max_len, w.split),
                                           dev)
        self.out = torch.empty((w.b, w.h_q, w.d), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((w.b, w.h_q), dtype=torch.float32, device=dev)
        self.bytes = decode_bytes(w, self.total)

    def run(self, i: int):
        import attention_forward_attn_amd as afa

        s = self.sets[i % len(self.sets)]
        afa.decode_paged_fp8(s["q"], s["k"], s["v"], self.k_scale, self.v_scale, self.table, self.kv_len,
                             self.max_len, scale=self.scale, sinks=self.sinks, split_size=self.w.split,
                             workspace=self.ws, out=self.out, lse=self.lse)


class BackwardCase:
    """dQ, dK, dV of the prefill for an incoming dO; O and LSE come from one forward outside the timing."""

    def __init__(self, w, n_sets: int, dev):
        import torch

        import attention_forward_attn_amd as afa
        from attention_forward_attn_amd.inputs import backward_inputs

        self.w = w
        base = backward_inputs(w.b, w.h_q, w.h_kv, w.s_q, w.s_k, w.d, w.seed)
        self.sets = [{n: base[n].to(dev) for n in ("q", "k", "v", "d_o")}]
        gen = torch.Generator(device=dev).manual_seed(w.seed + 1)
        for _ in range(1, n_sets):
            self.sets.append({n: torch.randn(t.shape, generator=gen, device=dev).to(torch.bfloat16)
                              for n, t in self.sets[0].items()})
        for st in self.sets:
            st["o"], st["lse"] = afa.prefill(st["q"], st["k"], st["v"], causal=w.causal)
        self.ws = torch.empty(afa.backward_workspace_size(w.b, w.h_q, w.s_q),
                              dtype=torch.uint8, device=dev)
        q, k = self.sets[0]["q"], self.sets[0]["k"]
        self.dq = torch.empty_like(q)
        self.dk = torch.empty_like(k)
        self.dv = torch.empty_like(k)
        # 2.5x the forward's count: five products (S, dP, dV, dQ, dK) of 2*d flops per visible pair
        self.flops = 10 * w.d * w.b * w.h_q * visible_pairs(w.s_q, w.s_k, w.causal, w.window)

    def run(self, i: int):
        import attention_forward_attn_amd as afa

        s = self.sets[i % len(self.sets)]
        afa.backward(s["q"], s["k"], s["v"], s["o"], s["d_o"], s["lse"], causal=self.w.causal, dq=self.dq,
                     dk=self.dk, dv=self.dv, workspace=self.ws)


def make_case(w, dev):
    """The bench case of a workload, rotating over enough input sets to defeat the MALL."""
    if w.kind == "backward":
        return BackwardCase(w, n_sets_beyond_mall(2 * prefill_set_bytes(w)), dev)
    if w.kind == "prefill":
        return PrefillCase(w, n_sets_beyond_mall(prefill_set_bytes(w)), dev)
    kind = (PagedFp8DecodeCase if w.fp8 and w.page_size else Fp8DecodeCase if w.fp8
            else PagedDecodeCase if w.page_size else DecodeCase)
    return kind(w, n_sets_beyond_mall(decode_set_bytes(w)), dev)


def bench_one(name: str, steps: int, warmup: int, dev, settle_s: float = 1.0):
    """One JSON line for one named workload alone (settle pass, warm-up, timed block)."""
    from attention_forward_attn_amd.inputs import WORKLOADS

    w = WORKLOADS[name]
    c = make_case(w, dev)
    st = settle(c, 0, min_s=settle_s) if settle_s > 0 else {"seconds": 0.0, "launches": 0}
    (ms,), wall = timed([c], steps, warmup, start=st["launches"])
    base = {"workload": name, "kind": w.kind, "ms": round(ms, 4), "input_sets": len(c.sets), "settle": st}
    if w.kind in ("prefill", "backward"):
        r = roofline_prefill(c.flops, ms)
        return {**base, "TFLOP/s": r["achieved"], "frac_of_peak": r["frac"], "gflop": round(c.flops / 1e9, 2)}
    r = roofline_decode(c.bytes, ms)
    return {**base, "GB/s": r["achieved"], "frac_of_peak": r["frac"], "MB": round(c.bytes / 1e6, 1)}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default=None, help="bench one named workload alone")
    ap.add_argument("--all", action="store_true", help="one line per workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--settle-seconds", type=float, default=1.0,
                    help="least duration of the clock-settle pass before the warm-up (0: no settle pass, e.g. "
                         "under a counter profiler, which serialises every launch)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 512 MiB device copy 3 times (a known-size reference for "
                         "HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this build runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(multi-GPU sharding is a design note, not built).", file=sys.stderr)
        sys.exit(2)

    import torch

    import attention_forward_attn_amd as afa
    from attention_forward_attn_amd.inputs import WORKLOADS

    afa.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_calibration:
        src = torch.ones(512 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.workload or args.all:
        names = [args.workload] if args.workload else list(WORKLOADS)
        for n in names:
            print(json.dumps(bench_one(n, args.steps, args.warmup, dev, args.settle_seconds)), flush=True)
        return

    wp = WORKLOADS[HEADLINE_PREFILL]
    wd = WORKLOADS[HEADLINE_DECODE]
    wd2 = WORKLOADS[SECOND_DECODE]
    pc, dc, dc2 = make_case(wp, dev), make_case(wd, dev), make_case(wd2, dev)
    # clock settle (time-based, before the warm-up steps), then warm-up and the timed steps
    st = settle(pc, 0, min_s=args.settle_seconds) if args.settle_seconds > 0 else {"seconds": 0.0, "launches": 0}
    start = st["launches"]
    (pre_ms, dec_ms, dec2_ms), wall_ms = timed([pc, dc, dc2], args.steps, args.warmup, start=start)
    start += args.warmup + args.steps
    pre = roofline_prefill(pc.flops, pre_ms, recorded_traffic(*PREFILL_PROFILE))
    dec = roofline_decode(dc.bytes, dec_ms, recorded_traffic(*DECODE_PROFILES[HEADLINE_DECODE]))
    dec2 = roofline_decode(dc2.bytes, dec2_ms, recorded_traffic(*DECODE_PROFILES[SECOND_DECODE]))
    n_spread = max(10, min(args.steps, 100))
    pre_spread = launch_spread(pc, n_spread, start)
    dec_spread = launch_spread(dc, n_spread, start)
    start += n_spread
    clock = clock_fraction(sampled_clock(pc, start, pre_ms), pre["achieved"])
    line = {
        "metric": "attn fwd TFLOPS (bf16, causal-adjusted) + decode HBM GB/s, 1xMI355X",
        "value": pre["achieved"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pre_ms + dec_ms + dec2_ms, 4),
        "wall_ms_per_step": round(wall_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic N(0,1) bf16, seeded",
        "config": {"workload": HEADLINE_PREFILL, "b": wp.b, "h_q": wp.h_q, "h_kv": wp.h_kv,
                   "s_q": wp.s_q, "s_k": wp.s_k, "d": wp.d, "causal": wp.causal,
                   "decode_workloads": [HEADLINE_DECODE, SECOND_DECODE], "decode_B": wd.b, "decode_h_q": wd.h_q,
                   "decode_h_kv": wd.h_kv, "decode_d": [wd.d, wd2.d], "decode_split": wd.split,
                   "decode_tokens": dc.total,
                   "step": "prefill, then decode at d=128, then decode at d=256",
                   "input_sets": {"prefill": len(pc.sets), "decode_d128": len(dc.sets),
                                  "decode_d256": len(dc2.sets)}},
        "settle": st,
        "prefill_ms": round(pre_ms, 4),
        "roofline": pre,
        "prefill_launch_spread": pre_spread,
        "prefill_clock": clock,
        "decode": {"value": dec["achieved"], "unit": "GB/s", "ms": round(dec_ms, 4),
                   "bytes": dc.bytes, "roofline": dec, "launch_spread": dec_spread},
        "decode_d256": {"value": dec2["achieved"], "unit": "GB/s", "ms": round(dec2_ms, 4),
                        "bytes": dc2.bytes, "roofline": dec2},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_prefill(wp)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
