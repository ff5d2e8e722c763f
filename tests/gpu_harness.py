"""Shared GPU-test plumbing: put a synthetic workload on the device, run the
library's store / plan / run on it through the C ABI, and compare against the
CPU oracle on the same seeded inputs."""

from __future__ import annotations

import sys

import numpy as np
import torch

import paged_kv_attention_store_amd as ak
from oracle import workload_run as orun
from synth import workloads as W

TOL = {  # max abs error bounds on out and lse
    "f32": (1e-4, 1e-4),
    "bf16": (2e-2, 1e-3),
    "fp8": (6e-2, 1e-3),
}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def prepare(wl: W.Workload, device="cuda", store_new=True):
    """Device tensors of the workload with the pool filled and (optionally) this
    step's new K/V stored.  FP8 pools are quantised by the library's own store."""
    d = W.device_inputs(wl, device)
    if wl.kv_dtype == "fp8":
        P, B, H, D = d["k_cache"].shape
        all_slots = torch.arange(P * B, dtype=torch.int64, device=device)
        ak.ak_store_kv(d["k_pool_src"].view(P * B, H, D), d["v_pool_src"].view(P * B, H, D),
                       all_slots, d["k_cache"], d["v_cache"], wl.kv_scale, wl.kv_scale)
        del d["k_pool_src"], d["v_pool_src"]
    if store_new:
        ak.ak_store_kv(d["k_new"], d["v_new"], d["slot_mapping"], d["k_cache"], d["v_cache"],
                       wl.kv_scale, wl.kv_scale)
    return d


def plan_for(wl: W.Workload, d, window, **kw):
    return ak.ak_plan(wl.qo_indptr, wl.kv_indptr, d["kv_indices"], wl.last_page_len,
                      wl.num_qo_heads, wl.num_kv_heads, wl.head_dim, wl.page_size,
                      causal=wl.causal, window=window, **kw)


def run(wl: W.Workload, d, plan, q=None):
    q = d["q"] if q is None else q
    lse = torch.full((wl.total_q, wl.num_qo_heads), float("nan"), dtype=torch.float32,
                     device=q.device)
    out = torch.full_like(q, float("nan"))
    ak.ak_run(plan, q, d["k_cache"], d["v_cache"], out=out, lse=lse, k_scale=wl.kv_scale,
              v_scale=wl.kv_scale)
    torch.cuda.synchronize()
    return out, lse


def rows_mask(wl: W.Workload, requests, rows_of=None):
    """Global query rows (tokens) covered by the sampled requests / rows."""
    sel = []
    for r in requests:
        q0, n = int(wl.qo_indptr[r]), int(wl.q_lens[r])
        js = np.arange(n) if rows_of is None else np.asarray(rows_of(r))
        sel.extend((q0 + js).tolist())
    return np.asarray(sorted(sel), dtype=np.int64)


def compare(wl: W.Workload, out, lse, window, requests=None, rows_of=None, caches=None):
    """Max |GPU - oracle| over the sampled rows; returns (err_out, err_lse, n_rows)."""
    if requests is None:
        requests = [r for r in range(wl.batch_size) if wl.q_lens[r] > 0]
    ref_o, ref_l = orun.run(wl, window=window, requests=requests, rows_of=rows_of, caches=caches)
    rows = rows_mask(wl, requests, rows_of)
    if len(rows) == 0:
        return 0.0, 0.0, 0
    go = out.float()[torch.from_numpy(rows).to(out.device)].cpu().numpy().astype(np.float64)
    gl = lse[torch.from_numpy(rows).to(out.device)].cpu().numpy().astype(np.float64)
    ro, rl = ref_o[rows], ref_l[rows]
    assert np.all(np.isfinite(go)), "non-finite output"
    assert np.all(np.isfinite(gl)), "non-finite lse"
    return float(np.max(np.abs(go - ro))), float(np.max(np.abs(gl - rl))), len(rows)


def check(wl: W.Workload, out, lse, window, **kw):
    eo, el, n = compare(wl, out, lse, window, **kw)
    tol_o, tol_l = TOL[wl.kv_dtype if wl.kv_dtype == "fp8" else wl.q_dtype]
    say(f"  {wl.name} window={window}: rows={n} max|dout|={eo:.3e} (tol {tol_o}) "
        f"max|dlse|={el:.3e} (tol {tol_l})")
    assert eo <= tol_o, f"out error {eo} > {tol_o}"
    assert el <= tol_l, f"lse error {el} > {tol_l}"
    return eo, el
