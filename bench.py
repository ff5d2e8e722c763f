"""Benchmark of the paged-KV attention hot path on one MI355X.

Headline step: one decode step of a Llama-3-8B-shaped model over a 64-request
batch (KV lengths uniform in [512, 8192], 32 q / 8 kv heads, head_dim 128, bf16,
page size 16, pages a random permutation of the pool): one ak_plan for the
batch, then for each of the 32 layers ak_store_kv of the 64 new K/V rows into
that layer's own cache followed by ak_run (split-KV decode + LSE merge).  All
inputs are resident in HBM before the timed region.

`value` = algorithmic HBM bytes of the step / step time (GB/s).
`tokens_per_s_per_layer` = the step's new query tokens over the step time per
layer (store, attention and merge; the plan amortised over the layers).  Algorithmic
bytes per layer = visible KV rows (K and V) + Q + out + lse + page ids read,
plus the store's reads and writes.  The roofline object reports the decode
attention kernel alone: its algorithmic bytes per launch over its average
duration from HIP events recorded, during the timed steps, around every launch
of that kernel on the launch stream (only the attention kernels carry events in
the timed steps; store and merge times come from a separate detail pass).

Further workloads (--also) are reported under their names: the ragged extend
batch ("prefill": large-tile kernel TFLOP/s against the bf16 dense MFMA peak),
the mixed chunked-prefill + decode step with full and sliding-window layers
("mixed"), the fp8 long-context decode ("longfp8"), decode requests sharing
a 4096-token prefix run plainly (with the shared-pages flag, and streamed) and
as a cascade ("cascade"), decode issued eagerly and as a replayed graph
over a fixed plan, on a small batch ("graph") and on the 64-request batch
above ("graph64"), and the decode and fp8 long-decode attention with the
split-KV plan against the stream-K plan ("streamk").
Two optional legs measure the large-tile kernel alone: on long uniform prompts
("prefill_shapes") and the fixed and per-block cost of a 256-row segment
("segcost").

The CPU baseline times the float64 oracle, after the GPU legs and in the same
run, on a bounded sample of each of the five workloads (decode in GB/s of the
same algorithmic bytes, extend in TFLOP/s of the same visible pairs, and tokens/s),
with the threads it used and the host's CPU count; the headline carries the
decode batch's figure, every other leg its own workload's.
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

METRIC = "paged decode attn HBM GB/s (% peak); prefill attn TFLOP/s (% MFMA peak)"

# Measured HBM traffic of the decode kernel (rocprofv3 FETCH_SIZE / WRITE_SIZE,
# scaled by the copy-kernel calibration) is kept with its profile summary, tagged
# with a hash of the sources the kernel is built from; it is reported only while
# those sources are unchanged.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_small_llama8b_decode_bf16.traffic.txt")
DECODE_KERNEL_SOURCES = [
    "paged_kv_attention_store_amd/csrc/ak_attn_small.hip",
    "paged_kv_attention_store_amd/csrc/ak_device.h",
    "paged_kv_attention_store_amd/csrc/ak_launch.h",
    "paged_kv_attention_store_amd/csrc/ak_internal.h",
    "paged_kv_attention_store_amd/csrc/ak_plan.cpp",   # the split decides the partial traffic
    "paged_kv_attention_store_amd/build.py",
]


def decode_kernel_sha() -> str:
    import hashlib

    h = hashlib.sha256()
    for rel in DECODE_KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per decode-kernel launch from the committed counter summary, or
    None when there is none or the kernel sources changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            kv = dict(line.split(":", 1) for line in f if ":" in line)
    except OSError:
        return None
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    if kv.get("sources_sha256") != decode_kernel_sha():
        return None
    return int(kv["fetch_bytes_per_launch"]) + int(kv["write_bytes_per_launch"])
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
EB = {"f32": 4, "bf16": 2, "fp8": 1}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ------------------------------------------------------- algorithmic work

def decode_bytes(wl, window=-1, small_only=False):
    """Algorithmic HBM bytes of one ak_run: visible KV rows (K and V), Q, out,
    lse and page ids.  `small_only` counts only requests whose rows per KV head
    (queries x group) fit a decode-shaped tile (<= 16)."""
    kv_tok = q_tok = pages = 0
    for r, (L, n) in enumerate(zip(wl.kv_lens, wl.q_lens)):
        L, n = int(L), int(n)
        if n == 0 or (small_only and n * wl.group > 16):
            continue
        kv_tok += L if window < 0 else min(L, window + n)
        q_tok += n
        pages += int(wl.kv_indptr[r + 1] - wl.kv_indptr[r])
    kv = kv_tok * wl.num_kv_heads * wl.head_dim * 2 * EB[wl.kv_dtype]
    qo = q_tok * wl.num_qo_heads * wl.head_dim * EB[wl.q_dtype] * 2
    return kv + qo + q_tok * wl.num_qo_heads * 4 + pages * 4


def store_bytes(wl):
    n = len(wl.slot_mapping)
    return n * wl.num_kv_heads * wl.head_dim * 2 * (EB[wl.q_dtype] + EB[wl.kv_dtype]) + 8 * n


def prefill_flops(wl, window=-1, large_only=False):
    """4 * D * Hq * (visible (query, key) pairs), causal/window aware.
    `large_only` counts only requests with more than 16 rows per KV head."""
    pairs = 0
    for L, n in zip(wl.kv_lens, wl.q_lens):
        L, n = int(L), int(n)
        if n == 0 or (large_only and n * wl.group <= 16):
            continue
        p = np.arange(L - n, L)
        lo = np.zeros_like(p) if window < 0 else np.maximum(0, p - window)
        pairs += int((p - lo + 1).sum())
    return 4.0 * wl.head_dim * wl.num_qo_heads * pairs


# ------------------------------------------------------------- device side

def make_layers(wl, n_layers, dev):
    """Per-layer caches (each its own pool), Q, new K/V and outputs on the device.
    FP8 pools are quantised from generated bf16 values by the library's store."""
    import torch

    import paged_kv_attention_store_amd as ak
    from synth import rng as R

    qd = torch.bfloat16 if wl.q_dtype == "bf16" else torch.float32
    shape = (wl.num_pages, wl.page_size, wl.num_kv_heads, wl.head_dim)
    flat = (wl.num_pages * wl.page_size, wl.num_kv_heads, wl.head_dim)
    layers = []
    for l in range(n_layers):
        s = wl.seed * 1000 + l
        if wl.kv_dtype == "fp8":
            kc = torch.empty(shape, dtype=torch.uint8, device=dev)
            vc = torch.empty(shape, dtype=torch.uint8, device=dev)
            ksrc = torch.empty(shape, dtype=torch.bfloat16, device=dev)
            vsrc = torch.empty(shape, dtype=torch.bfloat16, device=dev)
            R.fill_torch(ksrc, s, "k_pool")
            R.fill_torch(vsrc, s, "v_pool")
            all_slots = torch.arange(flat[0], dtype=torch.int64, device=dev)
            ak.ak_store_kv(ksrc.view(flat), vsrc.view(flat), all_slots, kc, vc, wl.kv_scale,
                           wl.kv_scale)
            torch.cuda.synchronize()
            del ksrc, vsrc, all_slots
        else:
            kc = torch.empty(shape, dtype=qd, device=dev)
            vc = torch.empty(shape, dtype=qd, device=dev)
            R.fill_torch(kc, s, "k_pool")
            R.fill_torch(vc, s, "v_pool")
        q = torch.empty(wl.total_q, wl.num_qo_heads, wl.head_dim, dtype=qd, device=dev)
        R.fill_torch(q, s, "q")
        kn = torch.empty(len(wl.slot_mapping), wl.num_kv_heads, wl.head_dim, dtype=qd, device=dev)
        vn = torch.empty_like(kn)
        R.fill_torch(kn, s, "k_new")
        R.fill_torch(vn, s, "v_new")
        out = torch.empty_like(q)
        lse = torch.empty(wl.total_q, wl.num_qo_heads, dtype=torch.float32, device=dev)
        layers.append(dict(kc=kc, vc=vc, q=q, kn=kn, vn=vn, out=out, lse=lse))
    return layers


def run_steps(ak, wl, layers, idx, slots, steps):
    """`steps` steps: one plan per window setting, then every layer stores its new
    K/V and runs with the plan of its window (layers alternate windows)."""
    plan_s = 0.0
    plans = None
    for _ in range(steps):
        t = time.perf_counter()
        plans = [ak.ak_plan(wl.qo_indptr, wl.kv_indptr, idx, wl.last_page_len, wl.num_qo_heads,
                            wl.num_kv_heads, wl.head_dim, wl.page_size, causal=wl.causal,
                            window=w) for w in wl.windows]
        plan_s += time.perf_counter() - t
        for i, L in enumerate(layers):
            ak.ak_store_kv(L["kn"], L["vn"], slots, L["kc"], L["vc"], wl.kv_scale, wl.kv_scale)
            ak.ak_run(plans[i % len(plans)], L["q"], L["kc"], L["vc"], out=L["out"], lse=L["lse"],
                      k_scale=wl.kv_scale, v_scale=wl.kv_scale)
    return plan_s, plans


def measure(ak, torch, dev, wl, n_layers, steps, warmup):
    """Time `steps` steps of the workload; per-kernel HIP-event times included."""
    log(f"[bench] {wl.name}: R={wl.batch_size} new tokens={wl.total_q} "
        f"KV tokens={int(wl.kv_lens.sum())} layers={n_layers} windows={wl.windows}")
    layers = make_layers(wl, n_layers, dev)
    idx = torch.from_numpy(wl.kv_indices.astype(np.int32)).to(dev)
    slots = torch.from_numpy(wl.slot_mapping).to(dev)
    torch.cuda.synchronize()
    run_steps(ak, wl, layers, idx, slots, warmup)
    torch.cuda.synchronize()
    # the timed steps carry HIP events around the attention kernels only (each
    # event pair adds a few microseconds between kernels); the store and merge
    # are timed in a separate detail pass
    G = wl.num_qo_heads // wl.num_kv_heads
    kinds = (["attn_small"] if np.any(wl.q_lens * G <= 16) else []) + \
            (["attn_large"] if np.any(wl.q_lens * G > 16) else [])
    ak.ak_profile_read()                      # reset counters
    ak.ak_profile_enable(True, kinds=kinds)
    t0 = time.perf_counter()
    plan_s, plans = run_steps(ak, wl, layers, idx, slots, steps)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ak.ak_profile_enable(False)
    prof = ak.ak_profile_read()
    ms_step = (t1 - t0) * 1e3 / steps
    detail_steps = max(2, steps // 2)
    ak.ak_profile_enable(True, kinds=["store_kv", "merge"])
    run_steps(ak, wl, layers, idx, slots, detail_steps)
    torch.cuda.synchronize()
    ak.ak_profile_enable(False)
    detail = ak.ak_profile_read()
    # host cost of planning alone; the in-step ak_plan calls also hold any wait
    # for a pooled workspace to come free when the host runs ahead of the GPU
    # (its last runs still executing), reported as the difference
    t = time.perf_counter()
    for _ in range(20):
        for w in wl.windows:
            ak.ak_plan(wl.qo_indptr, wl.kv_indptr, None, wl.last_page_len, wl.num_qo_heads,
                       wl.num_kv_heads, wl.head_dim, wl.page_size, causal=wl.causal, window=w,
                       host_only=True)
    plan_host_us = (time.perf_counter() - t) / 20 * 1e6
    wins = [wl.windows[i % len(wl.windows)] for i in range(n_layers)]
    dec_bytes = sum(decode_bytes(wl, w, small_only=True) for w in wins)
    flops = sum(prefill_flops(wl, w, large_only=True) for w in wins)
    step_bytes = sum(decode_bytes(wl, w) for w in wins) + n_layers * store_bytes(wl)
    res = dict(wl=wl, ms_step=ms_step, gbs=step_bytes / (ms_step * 1e-3) / 1e9, prof=prof,
               tok_s_layer=wl.total_q / (ms_step * 1e-3 / n_layers),
               dec_bytes=dec_bytes, flops=flops,
               info=ak.ak_plan_info(plans[0]), plan_call_us=plan_s / steps * 1e6,
               plan_host_us=plan_host_us,
               plan_wait_us=max(0.0, plan_s / steps * 1e6 - plan_host_us),
               step_bytes=step_bytes, layers=n_layers)
    n, ms = prof["attn_small"]
    if n and dec_bytes:
        res["small_avg_ms"] = ms / n
        res["small_bytes_per_launch"] = int(round(dec_bytes / n_layers))
        res["small_gbs"] = dec_bytes * steps / (ms * 1e-3) / 1e9
    n, ms = prof["attn_large"]
    if n and flops:
        res["large_avg_ms"] = ms / n
        res["large_tflops"] = flops * steps / (ms * 1e-3) / 1e12
    # both phases present: (bytes / HBM peak + flops / MFMA peak) over the measured
    # attention time of a step
    if "small_avg_ms" in res and "large_avg_ms" in res:
        t_att = n_layers * (res["small_avg_ms"] + res["large_avg_ms"]) * 1e-3
        res["combined_frac"] = (dec_bytes / (HBM_PEAK_GBS * 1e9) +
                                flops / (BF16_PEAK_TFLOPS * 1e12)) / t_att
    n, ms = detail["store_kv"]
    if n:
        res["store_avg_us"] = ms / n * 1e3
        res["store_gbs"] = store_bytes(wl) / (ms / n * 1e-3) / 1e9
    n, ms = detail["merge"]
    if n:
        res["merge_avg_us"] = ms / n * 1e3
    msg = (f"[bench] {wl.name}: {ms_step:.3f} ms/step, step-level {res['gbs']:.1f} GB/s; "
           f"plan {res['plan_host_us']:.1f} us host + {res['plan_wait_us']:.1f} us waiting for a "
           f"free workspace; ")
    if "small_gbs" in res:
        msg += f"attn_small {res['small_avg_ms'] * 1e3:.1f} us -> {res['small_gbs']:.1f} GB/s; "
    if "large_tflops" in res:
        msg += f"attn_large {res['large_avg_ms'] * 1e3:.1f} us -> {res['large_tflops']:.1f} TFLOP/s; "
    log(msg + f"profile {prof}; detail {detail}; plan {res['info']}")
    del layers
    torch.cuda.empty_cache()
    return res


def copy_bandwidth(torch, dev, gib):
    """Device-to-device copy of `gib` GiB (a plain copy kernel of known size):
    read + write bytes over the average time of 5 copies, as context for the
    HBM roofline."""
    n = int(gib * (1 << 30))
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 5
    gbs = 2 * n / (ms * 1e-3) / 1e9
    log(f"[bench] device copy of {gib} GiB: {ms * 1e3:.1f} us -> {gbs:.1f} GB/s (read + write)")
    del src, dst
    torch.cuda.empty_cache()
    return round(gbs, 1)


# ------------------------------------------------------------ CPU baseline

# Bounded samples of each workload for the oracle (request indices, seconds of
# timed passes).  The oracle's input generation is not timed.
CPU_SAMPLES = {
    1: ("all 4 decode requests", lambda wl: list(range(wl.batch_size)), 1.0),
    2: ("16 of 64 decode requests", lambda wl: list(range(16)), 8.0),
    3: ("2 of 8 extend requests", lambda wl: [0, 1], 6.0),
    4: ("the 2048-token chunk (request 0) and 8 of 255 decode requests, full attention",
        lambda wl: [0] + list(range(1, 9)), 8.0),
    5: ("1 of 8 decode requests (131072 KV tokens)", lambda wl: [0], 4.0),
}


def _host_cores():
    import threadpoolctl

    cpus = len(os.sched_getaffinity(0))
    blas = max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()] or [1])
    return cpus, blas


def _cpu_model():
    """The host CPU's model name, as the kernel reports it."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _cpu_leg(wl, reqs, budget_s, what):
    """Time the float64 oracle on `reqs` of `wl` (full attention) until `budget_s`
    seconds of passes; its algorithmic work in the GPU metric's unit."""
    from oracle import metadata as M
    from oracle import workload_run as orun

    kc, vc = orun.caches_after_store(wl)
    sl = np.concatenate([M.request_slots(wl.kv_indptr, wl.kv_indices, wl.last_page_len,
                                         wl.page_size, r) for r in reqs])
    kc.materialize(sl)          # input generation is not timed
    vc.materialize(sl)
    q = orun.decoded_q(wl)
    passes, t = 0, 0.0
    while t < budget_s or passes == 0:
        t0 = time.perf_counter()
        orun.run(wl, requests=reqs, caches=(kc, vc), q=q)
        t += time.perf_counter() - t0
        passes += 1
    sub = dict(q_lens=wl.q_lens[reqs], kv_lens=wl.kv_lens[reqs])
    tokens = int(sub["q_lens"].sum())
    if what == "decode":
        kv_tok = int(sub["kv_lens"].sum())
        work = kv_tok * wl.num_kv_heads * wl.head_dim * 2 * EB[wl.kv_dtype] + \
            tokens * wl.num_qo_heads * (wl.head_dim * EB[wl.q_dtype] * 2 + 4)
        value, unit = work * passes / t / 1e9, "GB/s"
    else:
        pairs = sum(int(n) * (int(L) - int(n)) + int(n) * (int(n) + 1) // 2
                    for n, L in zip(sub["q_lens"], sub["kv_lens"]))
        work = 4.0 * wl.head_dim * wl.num_qo_heads * pairs
        value, unit = work * passes / t / 1e12, "TFLOP/s"
    return value, unit, tokens * passes / t, passes, t


def cpu_baseline(k, wl=None):
    """The float64 oracle as it stands on a bounded sample of workload k, in the
    same algorithmic units as the GPU figure (decode GB/s, prefill TFLOP/s), on
    the host cores of this machine."""
    from synth import workloads as W

    wl = W.config(k) if wl is None else wl
    desc, pick, budget = CPU_SAMPLES[k]
    reqs = pick(wl)
    cpus, blas = _host_cores()
    legs = []
    if k == 4:
        legs.append(("prefill", [reqs[0]], budget / 2))
        legs.append(("decode", reqs[1:], budget / 2))
    else:
        legs.append(("prefill" if k == 3 else "decode", reqs, budget))
    out = []
    for what, rr, b in legs:
        value, unit, tok_s, passes, t = _cpu_leg(wl, rr, b, what)
        out.append({"value": round(value, 4), "unit": unit, "cores": int(blas), "host_cpus": cpus,
                    "cpu_model": _cpu_model(), "kind": "oracle", "phase": what,
                    "tokens_per_s": round(tok_s, 2), "wall_s_per_pass": round(t / passes, 3),
                    "sample": f"{wl.name}: {desc}; {what} part: requests {rr[:4]}"
                              f"{'...' if len(rr) > 4 else ''}, one layer, {passes} passes in "
                              f"{t:.1f} s; BLAS threads {blas} of {cpus} host CPUs"})
        log(f"[bench] cpu baseline config {k} ({what}): {value:.4f} {unit}, "
            f"{tok_s:.2f} tokens/s, {passes} passes in {t:.1f} s")
    return out[0] if len(out) == 1 else {o["phase"]: o for o in out}


# -------------------------------------------------------------------- main

def measure_cascade(ak, torch, dev, wl, n_layers, steps, warmup):
    """Shared-prefix decode two ways on the same caches: plain (one plan over every
    request's full page list) and cascade (the shared pages once for all queries
    as one non-causal request, each request's own pages, then ak_merge_states).
    Device time per layer from events on the stream, plans built beforehand."""
    log(f"[bench] {wl.name}: R={wl.batch_size} KV tokens={int(wl.kv_lens.sum())} "
        f"shared pages={wl.extra['shared_pages']} layers={n_layers}")
    layers = make_layers(wl, n_layers, dev)
    T, hq, hkv, D, B = wl.total_q, wl.num_qo_heads, wl.num_kv_heads, wl.head_dim, wl.page_size
    k = wl.extra["shared_pages"]
    idx = torch.from_numpy(wl.kv_indices.astype(np.int32)).to(dev)
    # plain decode twice: K/V streamed (the default) and with the shared-pages
    # flag (cached reads, so the shared prefix is served from the caches)
    plain_stream = ak.ak_plan(wl.qo_indptr, wl.kv_indptr, idx, wl.last_page_len, hq, hkv, D, B)
    plain = ak.ak_plan(wl.qo_indptr, wl.kv_indptr, idx, wl.last_page_len, hq, hkv, D, B,
                       shared_pages=True)
    idx_s = torch.from_numpy(wl.kv_indices[:k].astype(np.int32)).to(dev)
    shared = ak.ak_plan([0, T], [0, k], idx_s, [B], hq, hkv, D, B, causal=False)
    sx = np.concatenate([wl.kv_indices[wl.kv_indptr[r] + k:wl.kv_indptr[r + 1]]
                         for r in range(wl.batch_size)]).astype(np.int32)
    si = np.concatenate([[0], np.cumsum(np.diff(wl.kv_indptr) - k)]).astype(np.int32)
    idx_x = torch.from_numpy(sx).to(dev)
    suffix = ak.ak_plan(wl.qo_indptr, si, idx_x, wl.last_page_len, hq, hkv, D, B)
    o1, o2 = torch.empty_like(layers[0]["q"]), torch.empty_like(layers[0]["q"])
    l1 = torch.empty(T, hq, dtype=torch.float32, device=dev)
    l2 = torch.empty_like(l1)

    def plain_pass():
        for L in layers:
            ak.ak_run(plain, L["q"], L["kc"], L["vc"], out=L["out"], lse=L["lse"])

    def plain_stream_pass():
        for L in layers:
            ak.ak_run(plain_stream, L["q"], L["kc"], L["vc"], out=L["out"], lse=L["lse"])

    def cascade_pass():
        for L in layers:
            ak.ak_run(shared, L["q"], L["kc"], L["vc"], out=o1, lse=l1)
            ak.ak_run(suffix, L["q"], L["kc"], L["vc"], out=o2, lse=l2)
            ak.ak_merge_states(o1, l1, o2, l2, out=L["out"], lse_out=L["lse"])

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (steps * n_layers)

    plain_us, stream_us, cascade_us = timed(plain_pass), timed(plain_stream_pass), timed(cascade_pass)
    per_tok = hkv * D * 2 * EB[wl.kv_dtype]
    plain_bytes = decode_bytes(wl)
    cascade_bytes = plain_bytes - (wl.batch_size - 1) * k * B * per_tok
    res = {"workload": wl.name, "layers": n_layers, "shared_tokens": k * B,
           "plain_us_per_layer": round(plain_us, 1),
           "plain_streaming_us_per_layer": round(stream_us, 1),
           "cascade_us_per_layer": round(cascade_us, 1),
           "speedup": round(plain_us / cascade_us, 2),
           "plain_GBs": round(plain_bytes / (plain_us * 1e-6) / 1e9, 1),
           "cascade_GBs": round(cascade_bytes / (cascade_us * 1e-6) / 1e9, 1),
           "plain_bytes": plain_bytes, "cascade_bytes": cascade_bytes}
    log(f"[bench] {wl.name}: plain {plain_us:.1f} us/layer ({res['plain_GBs']} GB/s; "
        f"{stream_us:.1f} with streamed K/V), cascade "
        f"{cascade_us:.1f} us/layer ({res['cascade_GBs']} GB/s of its own bytes), "
        f"x{res['speedup']}")
    del layers
    torch.cuda.empty_cache()
    return res


def measure_graph(ak, torch, dev, wl, n_layers, steps, warmup, merge_in_kernel=True):
    """The same decode step (plan, then store_kv + run per layer) issued eagerly,
    and as a fixed plan updated on the host plus one replay of a graph holding
    every layer's store and run.  Wall time per step (host and device), the
    step's outputs compared bit for bit.  On a small batch launch cost dominates
    (there the parts of a split merge inside the attention kernel); on the
    64-request batch it shows what the gaps between launches cost (there the
    merge is its own launch, the faster choice at that size, as in the eager step)."""
    log(f"[bench] {wl.name}: R={wl.batch_size} KV tokens={int(wl.kv_lens.sum())} "
        f"layers={n_layers} (eager vs graph replay)")
    layers = make_layers(wl, n_layers, dev)
    idx = torch.from_numpy(wl.kv_indices.astype(np.int32)).to(dev)
    slots = torch.from_numpy(wl.slot_mapping).to(dev)
    hq, hkv, D, B = wl.num_qo_heads, wl.num_kv_heads, wl.head_dim, wl.page_size

    def eager_step():
        plan = ak.ak_plan(wl.qo_indptr, wl.kv_indptr, idx, wl.last_page_len, hq, hkv, D, B,
                          merge_in_kernel=merge_in_kernel)
        for L in layers:
            ak.ak_store_kv(L["kn"], L["vn"], slots, L["kc"], L["vc"])
            ak.ak_run(plan, L["q"], L["kc"], L["vc"], out=L["out"], lse=L["lse"])

    fixed = ak.ak_plan_fixed(wl.batch_size, wl.total_q, idx, hq, hkv, D, B,
                             max_query_len=int(wl.q_lens.max()), merge_in_kernel=merge_in_kernel)
    ak.ak_plan_update(fixed, wl.qo_indptr, wl.kv_indptr, wl.last_page_len)

    def body():
        for L in layers:
            ak.ak_store_kv(L["kn"], L["vn"], slots, L["kc"], L["vc"])
            ak.ak_run(fixed, L["q"], L["kc"], L["vc"], out=L["out"], lse=L["lse"])

    body()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        body()

    def graph_step():
        ak.ak_plan_update(fixed, wl.qo_indptr, wl.kv_indptr, wl.last_page_len)
        g.replay()

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e6 / steps

    eager_us, graph_us = timed(eager_step), timed(graph_step)
    eager_step()
    torch.cuda.synchronize()
    ref = [L["out"].clone() for L in layers]
    graph_step()
    torch.cuda.synchronize()
    same = all(torch.equal(r, L["out"]) for r, L in zip(ref, layers))
    step_bytes = n_layers * (decode_bytes(wl) + store_bytes(wl))
    res = {"workload": wl.name, "layers": n_layers, "requests": wl.batch_size,
           "kv_tokens": int(wl.kv_lens.sum()), "eager_us_per_step": round(eager_us, 1),
           "graph_us_per_step": round(graph_us, 1), "speedup": round(eager_us / graph_us, 2),
           "graph_step_GBs": round(step_bytes / (graph_us * 1e-6) / 1e9, 1),
           "merge_in_kernel": merge_in_kernel, "outputs_identical": bool(same),
           "capacity": {k: v for k, v in fixed.info().items() if k.startswith("cap_")}}
    log(f"[bench] {wl.name}: eager {eager_us:.1f} us/step, graph {graph_us:.1f} us/step "
        f"(x{res['speedup']}, {res['graph_step_GBs']} GB/s step-level), identical={same}")
    del layers, g
    torch.cuda.empty_cache()
    return res


def measure_stream_k(ak, torch, dev, launches=20):
    """Decode attention with the default split-KV plan and with the stream-K plan
    (equal contiguous shares of the decode KV, persistent workgroups) on the
    64-request decode batch and the fp8 long decode: average kernel time over
    `launches` runs alternating two layers' caches, HIP events on the stream."""
    from synth import workloads as W

    out = {}
    for k in (2, 5):
        wl = W.config(k)
        layers = make_layers(wl, 2, dev)
        idx = torch.from_numpy(wl.kv_indices.astype(np.int32)).to(dev)
        res = {}
        for name, kw in (("split_kv", {}), ("stream_k", {"stream_k": True})):
            plan = ak.ak_plan(wl.qo_indptr, wl.kv_indptr, idx, wl.last_page_len, wl.num_qo_heads,
                              wl.num_kv_heads, wl.head_dim, wl.page_size, **kw)
            for L in layers:
                ak.ak_run(plan, L["q"], L["kc"], L["vc"], out=L["out"], lse=L["lse"],
                          k_scale=wl.kv_scale, v_scale=wl.kv_scale)
            torch.cuda.synchronize()
            ak.ak_profile_read()
            ak.ak_profile_enable(True, kinds=["attn_small", "merge"])
            for i in range(launches):
                L = layers[i % 2]
                ak.ak_run(plan, L["q"], L["kc"], L["vc"], out=L["out"], lse=L["lse"],
                          k_scale=wl.kv_scale, v_scale=wl.kv_scale)
            torch.cuda.synchronize()
            ak.ak_profile_enable(False)
            pr = ak.ak_profile_read()
            us = pr["attn_small"][1] / pr["attn_small"][0] * 1e3
            mus = pr["merge"][1] / max(1, pr["merge"][0]) * 1e3
            info = ak.ak_plan_info(plan)
            res[name] = {"attn_us": round(us, 1), "merge_us": round(mus, 2),
                         "GBs": round(decode_bytes(wl) / ((us + mus) * 1e-6) / 1e9, 1),
                         "items": info["small_items"], "partial_rows": info["partial_rows"]}
            if name == "stream_k":
                res[name]["workgroups"] = info["stream_k_workgroups"]
        out[wl.name] = res
        log(f"[bench] {wl.name}: split-KV {res['split_kv']['attn_us']} + {res['split_kv']['merge_us']} us, "
            f"stream-K {res['stream_k']['attn_us']} + {res['stream_k']['merge_us']} us")
        del layers
        torch.cuda.empty_cache()
    return out


def time_large(ak, torch, dev, wl, launches=20):
    """Average duration (us) of the large-tile attention kernel on `wl`, HIP events
    around every launch, two layers with their own caches alternating."""
    layers = make_layers(wl, 2, dev)
    idx = torch.from_numpy(wl.kv_indices.astype(np.int32)).to(dev)
    plan = ak.ak_plan(wl.qo_indptr, wl.kv_indptr, idx, wl.last_page_len, wl.num_qo_heads,
                      wl.num_kv_heads, wl.head_dim, wl.page_size, causal=wl.causal, window=-1)
    for L in layers:
        ak.ak_run(plan, L["q"], L["kc"], L["vc"], out=L["out"], lse=L["lse"])
    torch.cuda.synchronize()
    ak.ak_profile_read()
    ak.ak_profile_enable(True, kinds=["attn_large"])
    for i in range(launches):
        L = layers[i % 2]
        ak.ak_run(plan, L["q"], L["kc"], L["vc"], out=L["out"], lse=L["lse"])
    torch.cuda.synchronize()
    ak.ak_profile_enable(False)
    n, ms = ak.ak_profile_read()["attn_large"]
    info = ak.ak_plan_info(plan)
    del layers, plan
    torch.cuda.empty_cache()
    return ms / n * 1e3, info["large_items"]


def measure_prefill_shapes(ak, torch, dev):
    """Large-tile kernel TFLOP/s on long uniform prompts (the kernel's steady state,
    against the ragged batch's short segments)."""
    from synth import workloads as W
    shapes = [
        ("8 x 2048 over 4096 cached, page 1", W.custom(11, [2048] * 8, [6144] * 8, 1, 32, 8, 128)),
        ("8 x 2048 over 4096 cached, page 16", W.custom(12, [2048] * 8, [6144] * 8, 16, 32, 8, 128)),
        ("1 x 16384, page 16", W.custom(13, [16384], [16384], 16, 32, 8, 128)),
        ("4 x 4096 non-causal, page 16",
         W.custom(14, [4096] * 4, [4096] * 4, 16, 32, 8, 128, causal=False)),
        ("8 x 1024, page 16", W.custom(15, [1024] * 8, [1024] * 8, 16, 32, 8, 128)),
    ]
    r3 = W.config(3)
    shapes.append(("ragged prefill batch, fp8 caches, page 16",
                   W.custom(16, r3.q_lens, r3.kv_lens, 16, 32, 8, 128, kv_dtype="fp8")))
    out = {}
    for name, wl in shapes:
        us, items = time_large(ak, torch, dev, wl)
        flops = prefill_flops(wl, -1) if wl.causal else \
            4.0 * wl.head_dim * wl.num_qo_heads * float(np.sum(wl.q_lens * wl.kv_lens))
        out[name] = {"segments": items, "avg_launch_us": round(us, 1),
                     "TFLOPs": round(flops / (us * 1e-6) / 1e12, 1)}
        log(f"[bench] prefill shape {name}: {items} segments, {us:.1f} us, "
            f"{out[name]['TFLOPs']} TFLOP/s")
    return out


def measure_segcost(ak, torch, dev, cus=256):
    """Fixed and per-block cost of one 256-row segment: 256 requests of 64 new tokens
    (one segment per KV head, 8 segments per compute unit) over KV lengths of k
    blocks of 128 tokens, fitted as time per segment = fixed + k * per_block."""
    from synth import workloads as W
    ks, per_seg = [], []
    for k in (1, 2, 4, 8, 16, 32):
        wl = W.custom(20 + k, [64] * 256, [128 * k] * 256, 16, 32, 8, 128)
        us, items = time_large(ak, torch, dev, wl)
        ks.append(k)
        per_seg.append(us / (items / cus))
        log(f"[bench] segment cost: {k} blocks per segment, {items} segments, {us:.1f} us per launch, "
            f"{per_seg[-1]:.2f} us per segment per CU")
    A = np.vstack([np.ones(len(ks)), np.array(ks, float)]).T
    (fixed, per_block), *_ = np.linalg.lstsq(A, np.array(per_seg), rcond=None)
    log(f"[bench] segment cost fit: {fixed:.2f} us fixed + {per_block:.3f} us per block")
    return {"blocks": ks, "us_per_segment_per_cu": [round(x, 2) for x in per_seg],
            "fixed_us": round(float(fixed), 2), "per_block_us": round(float(per_block), 3)}


WORKLOADS = {
    # name: (factory, layers with distinct caches)
    "prefill": (lambda W: W.config(3), 2),
    "mixed": (lambda W: W.config(4), 4),
    "longfp8": (lambda W: W.config(5), 4),
    "cascade": (lambda W: W.shared_prefix_decode(), 8),
    "graph": (lambda W: W.small_batch_decode(), 32),
    "graph64": (lambda W: W.config(2), 32),
    "prefill_shapes": (None, 2),
    "segcost": (None, 2),
    "streamk": (None, 2),
}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=32, help="layers of the headline decode step")
    ap.add_argument("--also", default="prefill,mixed,longfp8,cascade,graph,graph64,streamk",
                    help="comma list of further workloads: prefill,mixed,longfp8,cascade,graph,"
                         "graph64,streamk (default), prefill_shapes, segcost ('' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-gib", type=float, default=1.0,
                    help="size of the device-to-device copy timed as bandwidth context (0: skip)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only; there is no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import paged_kv_attention_store_amd as ak
    from synth import workloads as W

    dev = torch.device("cuda:0")
    copy = copy_bandwidth(torch, dev, args.copy_gib) if args.copy_gib > 0 else None
    dec = measure(ak, torch, dev, W.config(2), args.layers, args.steps, args.warmup)
    extra = {}
    for name in [x for x in args.also.split(",") if x]:
        fac, nl = WORKLOADS[name]
        if name == "cascade":
            extra[name] = measure_cascade(ak, torch, dev, fac(W), nl, max(2, args.steps), 2)
            continue
        if name in ("graph", "graph64"):
            extra[name] = measure_graph(ak, torch, dev, fac(W), nl, max(5, args.steps), 3,
                                        merge_in_kernel=name == "graph")
            continue
        if name == "prefill_shapes":
            extra[name] = measure_prefill_shapes(ak, torch, dev)
            continue
        if name == "segcost":
            extra[name] = measure_segcost(ak, torch, dev)
            continue
        if name == "streamk":
            extra[name] = measure_stream_k(ak, torch, dev)
            continue
        extra[name] = measure(ak, torch, dev, fac(W), nl, max(2, args.steps), 2)
    # the oracle on a bounded sample of every workload (configs 1-5), after the
    # GPU legs, in this same run
    cpu_by = {} if args.no_cpu_baseline else {k: cpu_baseline(k) for k in (1, 2, 3, 4, 5)}
    cpu = cpu_by.get(2)
    leg_config = {"prefill": 3, "mixed": 4, "longfp8": 5}
    traffic = measured_traffic()
    wl = dec["wl"]
    line = {
        "metric": METRIC,
        "value": round(dec["gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["ms_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "llama8b-shaped batched decode: 64 requests, KV lengths U[512,8192], "
                        "32 q / 8 kv heads, head_dim 128, bf16, page 16, random page permutation; "
                        f"step = 1 plan + {args.layers} layers x (store_kv of 64 tokens + run)",
            "layers": args.layers,
            "kv_tokens": int(wl.kv_lens.sum()),
            "bytes_per_step": dec["step_bytes"],
            "plan_host_us": round(dec["plan_host_us"], 1),
            "plan_wait_us": round(dec["plan_wait_us"], 1),
            "plan": dec["info"],
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "attn_small (decode, split-KV)",
            "achieved": round(dec["small_gbs"], 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(dec["small_gbs"] / HBM_PEAK_GBS, 4),
            "avg_launch_us": round(dec["small_avg_ms"] * 1e3, 2),
            "algorithmic_bytes_per_launch": dec["small_bytes_per_launch"],
            "traffic": traffic,
        },
        "cpu_baseline": cpu,
        "cpu_baseline_by_config": {str(k): v for k, v in cpu_by.items()},
        "copy_GBs": copy,
        "tokens_per_s_per_layer": round(dec["tok_s_layer"], 1),
    }
    for name, r in extra.items():
        if name in ("cascade", "graph", "graph64", "prefill_shapes", "segcost", "streamk"):
            line[name] = r
            continue
        e = {"workload": r["wl"].name, "ms_per_step": round(r["ms_step"], 4),
             "layers": r["layers"], "step_GBs": round(r["gbs"], 1),
             "plan_host_us": round(r["plan_host_us"], 1), "plan_wait_us": round(r["plan_wait_us"], 1),
             "tokens_per_s_per_layer": round(r["tok_s_layer"], 1)}
        if "small_gbs" in r:
            e["decode"] = {"kernel": "attn_small", "achieved": round(r["small_gbs"], 1),
                           "unit": "GB/s", "peak": HBM_PEAK_GBS,
                           "frac": round(r["small_gbs"] / HBM_PEAK_GBS, 4),
                           "avg_launch_us": round(r["small_avg_ms"] * 1e3, 2)}
        if "large_tflops" in r:
            e["prefill"] = {"kernel": "attn_large", "achieved": round(r["large_tflops"], 2),
                            "unit": "TFLOP/s", "peak": BF16_PEAK_TFLOPS,
                            "frac": round(r["large_tflops"] / BF16_PEAK_TFLOPS, 4),
                            "avg_launch_us": round(r["large_avg_ms"] * 1e3, 2)}
        if "store_gbs" in r:
            e["store_kv"] = {"GBs": round(r["store_gbs"], 1), "avg_us": round(r["store_avg_us"], 2)}
        if "merge_avg_us" in r:
            e["merge_avg_us"] = round(r["merge_avg_us"], 2)
        if "combined_frac" in r:
            e["combined_roofline_frac"] = round(r["combined_frac"], 4)
        if name in leg_config and leg_config[name] in cpu_by:
            e["cpu_baseline"] = cpu_by[leg_config[name]]
        line[name] = e
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
