"""Seeded random batches over the documented parameter ranges, on the GPU against
the fp64 CPU oracle element by element: page sizes 1/16/64, GQA groups 1 to 16,
head dims 64/128, bf16 and fp8 caches, causal or not, with and without a sliding
window, each request a decode, a short multi-row query, an empty query or an
extend chunk, each batch planned plainly and with forced KV splits (merge
launched, or merged inside the attention kernel).  The hand-picked edge cases
cover single features; these mix them.  The CPU test checks that the host
planner accepts every drawn batch, so a GPU run only meets batches the planner
has already seen."""

import numpy as np
import pytest

import paged_kv_attention_store_amd as ak
from synth import workloads as W

SEEDS = list(range(16))
HEADS = [(8, 8), (8, 2), (32, 8), (16, 1), (64, 8)]


def draw(seed: int):
    """One batch: (name, q_lens, kv_lens, page size, hq, hkv, D, kv dtype, causal,
    windows, forced-split options)."""
    rng = np.random.default_rng(7000 + seed)
    R = int(rng.integers(1, 7))
    B = int(rng.choice([1, 16, 64]))
    hq, hkv = HEADS[int(rng.integers(len(HEADS)))]
    D = int(rng.choice([64, 128]))
    kd = "fp8" if rng.random() < 0.5 else "bf16"
    causal = bool(rng.random() < 0.8)
    q_lens, kv_lens = [], []
    for _ in range(R):
        u = rng.random()
        if u < 0.45:
            q = 1
        elif u < 0.6:
            q = int(rng.integers(2, 5))
        elif u < 0.7:
            q = 0
        else:
            q = int(rng.integers(5, 65))
        kv = q + int(rng.integers(0 if q else 1, 1200))
        q_lens.append(q)
        kv_lens.append(kv)
    wdraw = (rng.random(), int(rng.integers(0, 300)))
    # a sliding window is defined for causal attention only (the planner rejects it otherwise)
    windows = (-1, wdraw[1]) if causal and wdraw[0] >= 0.5 else (-1,)
    split = {"min_chunk": 64, "num_cus": 1024, "merge_in_kernel": bool(rng.random() < 0.5)}
    name = f"rand{seed}_B{B}_h{hq}x{hkv}_D{D}_{kd}_{'c' if causal else 'nc'}"
    return name, q_lens, kv_lens, B, hq, hkv, D, kd, causal, windows, split


def workload(seed: int):
    name, ql, kl, B, hq, hkv, D, kd, causal, windows, split = draw(seed)
    wl = W.custom(seed=9000 + seed, q_lens=ql, kv_lens=kl, page_size=B, num_qo_heads=hq,
                  num_kv_heads=hkv, head_dim=D, q_dtype="bf16", kv_dtype=kd, causal=causal,
                  windows=windows, name=name)
    return wl, windows, split


@pytest.mark.parametrize("seed", SEEDS)
def test_random_batch_plans_on_host(seed):
    wl, windows, split = workload(seed)
    for window in windows:
        for kw in ({}, split):
            plan = ak.ak_plan(wl.qo_indptr, wl.kv_indptr, None, wl.last_page_len,
                              wl.num_qo_heads, wl.num_kv_heads, wl.head_dim, wl.page_size,
                              causal=wl.causal, window=window, host_only=True, **kw)
            info = ak.ak_plan_info(plan)
            assert info["batch_size"] == wl.batch_size and info["total_q"] == wl.total_q
            assert info["items"] == info["small_items"] + info["large_items"]
            assert (info["items"] > 0) == (wl.total_q > 0)


@pytest.mark.gpu
@pytest.mark.parametrize("seed", SEEDS)
def test_random_batch_parity(seed):
    from tests.gpu_harness import check, plan_for, prepare, run, say

    wl, windows, split = workload(seed)
    say(f"[random] {wl.name} q={wl.q_lens.tolist()} kv={wl.kv_lens.tolist()} "
        f"windows={windows} split={split}")
    d = prepare(wl)
    for window in windows:
        for kw in ({}, split):
            plan = plan_for(wl, d, window, **kw)
            out, lse = run(wl, d, plan)
            check(wl, out, lse, window)


# Longer batches: extend chunks of up to 1536 tokens on prefixes of up to 3000, so
# a (request, KV head) spans several 256-row segments and many 128-token KV blocks
# (the reference max raised inside long block runs, segments grouped by die when
# the batch has few units, KV splits of long segments); page sizes up to 128.
# Compared on sampled rows: the first and last three of each request and 26 drawn.
LONG_SEEDS = list(range(12))


def draw_long(seed: int):
    rng = np.random.default_rng(8100 + seed)
    R = int(rng.integers(1, 5))
    B = int(rng.choice([1, 2, 16, 64, 128]))
    hq, hkv = HEADS[int(rng.integers(len(HEADS)))]
    D = int(rng.choice([64, 128]))
    kd = "fp8" if rng.random() < 0.4 else "bf16"
    causal = bool(rng.random() < 0.85)
    q_lens, kv_lens = [], []
    for _ in range(R):
        q = 1 if rng.random() < 0.2 else int(rng.integers(65, 1537))
        prefix = int(rng.integers(0, 3001))
        q_lens.append(q)
        kv_lens.append(q + prefix)
    windows = (-1, int(rng.integers(64, 2049))) if causal and rng.random() < 0.5 else (-1,)
    split = {"min_chunk": 128, "num_cus": int(rng.choice([64, 1024])),
             "merge_in_kernel": bool(rng.random() < 0.5)}
    name = f"long{seed}_B{B}_h{hq}x{hkv}_D{D}_{kd}_{'c' if causal else 'nc'}"
    wl = W.custom(seed=9500 + seed, q_lens=q_lens, kv_lens=kv_lens, page_size=B,
                  num_qo_heads=hq, num_kv_heads=hkv, head_dim=D, q_dtype="bf16", kv_dtype=kd,
                  causal=causal, windows=windows, name=name)
    return wl, windows, split


def _sampled_rows(wl, seed):
    rng = np.random.default_rng(8200 + seed)
    rows = {}
    for r in range(wl.batch_size):
        n = int(wl.q_lens[r])
        pick = set(range(min(3, n))) | set(range(max(0, n - 3), n))
        pick |= set(rng.integers(0, n, size=min(26, n)).tolist()) if n else set()
        rows[r] = sorted(pick)
    return rows


@pytest.mark.parametrize("seed", LONG_SEEDS)
def test_long_random_batch_plans_on_host(seed):
    wl, windows, split = draw_long(seed)
    for window in windows:
        for kw in ({}, split):
            plan = ak.ak_plan(wl.qo_indptr, wl.kv_indptr, None, wl.last_page_len,
                              wl.num_qo_heads, wl.num_kv_heads, wl.head_dim, wl.page_size,
                              causal=wl.causal, window=window, host_only=True, **kw)
            info = ak.ak_plan_info(plan)
            assert info["batch_size"] == wl.batch_size and info["total_q"] == wl.total_q


@pytest.mark.gpu
@pytest.mark.parametrize("seed", LONG_SEEDS)
def test_long_random_batch_parity(seed):
    from tests.gpu_harness import check, plan_for, prepare, run, say

    wl, windows, split = draw_long(seed)
    say(f"[random-long] {wl.name} q={wl.q_lens.tolist()} kv={wl.kv_lens.tolist()} "
        f"windows={windows} split={split}")
    rows = _sampled_rows(wl, seed)
    d = prepare(wl)
    for window in windows:
        for kw in ({}, split):
            plan = plan_for(wl, d, window, **kw)
            out, lse = run(wl, d, plan)
            check(wl, out, lse, window, rows_of=lambda r: rows[r])
