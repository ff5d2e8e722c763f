"""Benchmark of the paged-KV attention hot path on one MI355X.

A step is one decode step of a Llama-3-8B-shaped model over a 64-request batch
(KV lengths uniform in [512, 8192], 32 q / 8 kv heads, head_dim 128, bf16,
page size 16, pages a random permutation of the pool): one ak_plan for the
batch, then for each of the 32 layers ak_store_kv of the 64 new K/V rows into
that layer's own cache followed by ak_run (split-KV decode + LSE merge).  All
inputs are resident in HBM before the timed region.

`value` = algorithmic HBM bytes of the step / step time (GB/s).  Algorithmic
bytes per layer = visible KV (K and V) + Q + out + lse + page ids read, plus
the store's read and write.  The roofline object reports the decode attention
kernel alone: its algorithmic bytes per launch over its average duration from
HIP events recorded around every launch on the launch stream.

A second measurement (reported under "prefill") runs the ragged extend batch
(8 requests, 128..2048 new tokens over a 0..4096-token prefix, page size 1) and
reports the large-tile kernel's TFLOP/s against the bf16 dense MFMA peak.

The CPU baseline times the float64 oracle on a sample of the same decode batch.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode attn HBM GB/s (% peak); prefill attn TFLOP/s (% MFMA peak)"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def decode_bytes(wl, window=-1):
    """Algorithmic HBM bytes of one ak_run over the batch."""
    eb = {"f32": 4, "bf16": 2, "fp8": 1}
    kv_tok = 0
    for L, n in zip(wl.kv_lens, wl.q_lens):
        if n == 0:
            continue
        vis = int(L) if window < 0 else min(int(L), window + int(n))
        kv_tok += vis
    kv = kv_tok * wl.num_kv_heads * wl.head_dim * 2 * eb[wl.kv_dtype]
    qo = wl.total_q * wl.num_qo_heads * wl.head_dim * eb[wl.q_dtype] * 2
    lse = wl.total_q * wl.num_qo_heads * 4
    idx = int(wl.kv_indptr[-1]) * 4
    return kv + qo + lse + idx


def store_bytes(wl):
    eb = {"f32": 4, "bf16": 2, "fp8": 1}
    n = len(wl.slot_mapping)
    per = wl.num_kv_heads * wl.head_dim * 2
    return n * per * (eb[wl.q_dtype] + eb[wl.kv_dtype]) + 8 * n


def prefill_flops(wl, window=-1):
    """4 * D * Hq * (visible (query, key) pairs), causal/window aware."""
    pairs = 0
    for L, n in zip(wl.kv_lens, wl.q_lens):
        L, n = int(L), int(n)
        for j in range(n):
            p = L - n + j
            lo = 0 if window < 0 else max(0, p - window)
            pairs += p - lo + 1
    return 4.0 * wl.head_dim * wl.num_qo_heads * pairs


def make_layers(wl, n_layers, dev):
    import torch

    from synth import rng as R

    qd = torch.bfloat16 if wl.q_dtype == "bf16" else torch.float32
    shape = (wl.num_pages, wl.page_size, wl.num_kv_heads, wl.head_dim)
    layers = []
    for l in range(n_layers):
        s = wl.seed * 1000 + l
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


def run_steps(ak, wl, layers, idx, slots, steps, window=-1):
    import torch

    plan_s = 0.0
    for _ in range(steps):
        t = time.perf_counter()
        plan = ak.ak_plan(wl.qo_indptr, wl.kv_indptr, idx, wl.last_page_len, wl.num_qo_heads,
                          wl.num_kv_heads, wl.head_dim, wl.page_size, causal=wl.causal,
                          window=window)
        plan_s += time.perf_counter() - t
        for L in layers:
            ak.ak_store_kv(L["kn"], L["vn"], slots, L["kc"], L["vc"])
            ak.ak_run(plan, L["q"], L["kc"], L["vc"], out=L["out"], lse=L["lse"])
    return plan_s, plan


def bench_decode(args, ak, torch, dev):
    from synth import workloads as W

    wl = W.config(2)
    log(f"[bench] decode workload {wl.name}: R={wl.batch_size} KV tokens={int(wl.kv_lens.sum())} "
        f"layers={args.layers}")
    layers = make_layers(wl, args.layers, dev)
    idx = torch.from_numpy(wl.kv_indices.astype(np.int32)).to(dev)
    slots = torch.from_numpy(wl.slot_mapping).to(dev)
    torch.cuda.synchronize()
    run_steps(ak, wl, layers, idx, slots, args.warmup)
    torch.cuda.synchronize()
    ak.ak_profile_read()                      # reset counters
    ak.ak_profile_enable(True)
    t0 = time.perf_counter()
    plan_s, plan = run_steps(ak, wl, layers, idx, slots, args.steps)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ak.ak_profile_enable(False)
    prof = ak.ak_profile_read()
    info = ak.ak_plan_info(plan)
    ms_step = (t1 - t0) * 1e3 / args.steps
    b_layer = decode_bytes(wl) + store_bytes(wl)
    step_bytes = args.layers * b_layer
    gbs = step_bytes / (ms_step * 1e-3) / 1e9
    n_att, ms_att = prof["attn_small"]
    att_avg_ms = ms_att / max(n_att, 1)
    att_gbs = decode_bytes(wl) / (att_avg_ms * 1e-3) / 1e9
    log(f"[bench] decode: {ms_step:.3f} ms/step, {gbs:.1f} GB/s step-level; attn_small avg "
        f"{att_avg_ms * 1e3:.1f} us -> {att_gbs:.1f} GB/s; plan {plan_s / args.steps * 1e6:.1f} us; "
        f"profile {prof}; plan info {info}")
    return dict(wl=wl, ms_step=ms_step, gbs=gbs, att_avg_ms=att_avg_ms, att_gbs=att_gbs,
                prof=prof, info=info, plan_us=plan_s / args.steps * 1e6, b_layer=b_layer)


def bench_prefill(args, ak, torch, dev):
    from synth import workloads as W

    wl = W.config(3)
    flops = prefill_flops(wl)
    log(f"[bench] prefill workload {wl.name}: new tokens={wl.total_q} flops={flops / 1e9:.1f} G")
    layers = make_layers(wl, 2, dev)
    idx = torch.from_numpy(wl.kv_indices.astype(np.int32)).to(dev)
    slots = torch.from_numpy(wl.slot_mapping).to(dev)
    run_steps(ak, wl, layers, idx, slots, 2)
    torch.cuda.synchronize()
    ak.ak_profile_read()
    ak.ak_profile_enable(True)
    steps = max(2, args.steps // 2)
    t0 = time.perf_counter()
    run_steps(ak, wl, layers, idx, slots, steps)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ak.ak_profile_enable(False)
    prof = ak.ak_profile_read()
    n, ms = prof["attn_large"]
    avg = ms / max(n, 1)
    tflops = flops / (avg * 1e-3) / 1e12
    ns, mss = prof["store_kv"]
    st_avg = mss / max(ns, 1)
    st_gbs = store_bytes(wl) / (st_avg * 1e-3) / 1e9
    log(f"[bench] prefill: attn_large avg {avg * 1e3:.1f} us -> {tflops:.1f} TFLOP/s; "
        f"store_kv avg {st_avg * 1e3:.1f} us -> {st_gbs:.1f} GB/s; step {(t1 - t0) * 1e3 / steps / 2:.3f} ms/layer")
    return dict(tflops=tflops, avg_ms=avg, flops=flops, store_gbs=st_gbs, store_us=st_avg * 1e3)


def cpu_baseline(wl, budget_s=12.0, n_req=16):
    """The float64 oracle as it stands, on a sample of the decode batch."""
    import threadpoolctl

    from oracle import metadata as M
    from oracle import workload_run as orun

    reqs = list(range(n_req))
    kc, vc = orun.caches_after_store(wl)
    sl = np.concatenate([M.request_slots(wl.kv_indptr, wl.kv_indices, wl.last_page_len,
                                         wl.page_size, r) for r in reqs])
    kc.materialize(sl)
    vc.materialize(sl)
    q = orun.decoded_q(wl)
    sub = dict(kv_lens=wl.kv_lens[reqs])
    kv_bytes = int(sub["kv_lens"].sum()) * wl.num_kv_heads * wl.head_dim * 2 * 2
    qo = n_req * wl.num_qo_heads * wl.head_dim * 2 * 2
    passes, t = 0, 0.0
    while t < budget_s:
        t0 = time.perf_counter()
        orun.run(wl, requests=reqs, caches=(kc, vc), q=q)
        t += time.perf_counter() - t0
        passes += 1
    threads = max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()] or [1])
    gbs = (kv_bytes + qo) * passes / t / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n_req} of {wl.batch_size} decode requests ({int(sub['kv_lens'].sum())} KV "
                      f"tokens), one layer, {passes} passes in {t:.1f} s; host cores available "
                      f"{len(os.sched_getaffinity(0))}"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import paged_kv_attention_store_amd as ak

    dev = torch.device("cuda:0")
    dec = bench_decode(args, ak, torch, dev)
    pre = None if args.no_prefill else bench_prefill(args, ak, torch, dev)
    cpu = None if args.no_cpu_baseline else cpu_baseline(dec["wl"])
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
            "bytes_per_layer": dec["b_layer"],
            "plan_us": round(dec["plan_us"], 1),
            "plan": dec["info"],
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "attn_small (decode, split-KV)",
            "achieved": round(dec["att_gbs"], 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(dec["att_gbs"] / HBM_PEAK_GBS, 4),
            "avg_launch_us": round(dec["att_avg_ms"] * 1e3, 2),
            "traffic": None,
        },
        "cpu_baseline": cpu,
    }
    if pre is not None:
        line["prefill"] = {
            "workload": "ragged extend: 8 requests, 128..2048 new tokens over 0..4096 prefix, "
                        "32/8 heads, head_dim 128, bf16, page size 1",
            "kernel": "attn_large",
            "achieved": round(pre["tflops"], 2),
            "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(pre["tflops"] / BF16_PEAK_TFLOPS, 4),
            "avg_launch_us": round(pre["avg_ms"] * 1e3, 2),
            "gflop_per_launch": round(pre["flops"] / 1e9, 2),
            "store_kv_GBs": round(pre["store_gbs"], 1),
            "store_kv_us": round(pre["store_us"], 2),
        }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
