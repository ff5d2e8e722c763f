"""Attention on the GPU against the fp64 CPU oracle, element by element on the
same seeded inputs: the five workloads at reduced sizes (full comparison), at
their full sizes (sampled requests / query rows, in the launch configuration
the benchmark times), and edge cases."""

import numpy as np
import pytest
import torch

import paged_kv_attention_store_amd as ak
from synth import rng as R
from synth import workloads as W
from tests.gpu_harness import check, plan_for, prepare, run, say

pytestmark = pytest.mark.gpu


def _full(wl, windows=None, **plan_kw):
    d = prepare(wl)
    for window in (windows or wl.windows):
        plan = plan_for(wl, d, window, **plan_kw)
        say(f"[parity] {wl.name} {ak.ak_plan_info(plan)}")
        out, lse = run(wl, d, plan)
        check(wl, out, lse, window)


# ------------------------------------------------ reduced-size workloads

def test_tiny_decode_fp32():
    _full(W.config(1))


def test_decode_bf16_reduced():
    _full(W.llama8b_decode(seed=2, R=8))


def test_prefill_bf16_reduced():
    _full(W.ragged_prefill(seed=3, R=4, n_range=(100, 300), p_range=(0, 600)))


def test_mixed_bf16_reduced():
    wl = W.mixed_chunk_decode(seed=4, R_dec=40, chunk=300, prefix=700, lmin=100, lmax=6000)
    _full(wl, windows=(-1, 4096, 256))


def test_mixed_bf16_reduced_shuffled():
    wl = W.mixed_chunk_decode(seed=4, R_dec=40, chunk=300, prefix=700, lmin=100, lmax=6000,
                              shuffle=True)
    _full(wl, windows=(-1, 256))


def test_long_decode_fp8_reduced():
    _full(W.llama70b_long_decode(seed=5, R=2, L=20000))


# ---------------------------------------------- full sizes, sampled checks

def _sample_rows(wl, r, k=24, window=-1):
    """Query rows of request r to compare: all of a short request; otherwise the
    first and last rows, the middle, k random rows, rows either side of every
    64-token boundary (a 256-row large tile holds 64 query tokens at group 4)
    and, with a window, rows whose window start crosses a 128-token KV block."""
    n = int(wl.q_lens[r])
    if n <= k:
        return np.arange(n)
    rng = np.random.default_rng(r)
    pick = set([0, 1, n // 2, n - 2, n - 1]) | set(rng.choice(n, size=k, replace=False).tolist())
    for b in range(64, n, 64 * max(1, n // 1024)):
        pick |= {b - 1, b}
    if window >= 0:
        L = int(wl.kv_lens[r])
        start = L - n + np.arange(n) - window          # first visible key of each row
        cross = np.nonzero((start > 0) & (start % 128 == 0))[0]
        for j in cross[:: max(1, len(cross) // 8)]:
            pick |= {int(j) - 1, int(j), int(j) + 1}
    return np.asarray(sorted(x for x in pick if 0 <= x < n))


def _full_size_requests(wl, k):
    """Requests compared at full size: the longest, the shortest, a few random
    ones and every request with more than one query row."""
    order = np.argsort(-wl.kv_lens)
    if k == 5:
        reqs = {int(order[0]), int(order[-1])}
    else:
        rng = np.random.default_rng(k)
        reqs = set(order[:3].tolist()) | set(order[-2:].tolist()) | \
            set(rng.choice(wl.batch_size, size=min(6, wl.batch_size), replace=False).tolist())
    reqs |= set(np.nonzero(wl.q_lens > 1)[0].tolist())
    return sorted(int(r) for r in reqs)


def _check_full_size(wl, k):
    say(f"[parity-full] {wl.name} (config {k}): R={wl.batch_size} tokens={wl.total_q} "
        f"kv={int(wl.kv_lens.sum())}")
    d = prepare(wl)
    reqs = _full_size_requests(wl, k)
    say(f"  compared requests {reqs}")
    for window in wl.windows:
        plan = plan_for(wl, d, window)
        say(f"  plan {ak.ak_plan_info(plan)}")
        out, lse = run(wl, d, plan)
        check(wl, out, lse, window, requests=reqs,
              rows_of=lambda r, w=window: _sample_rows(wl, r, window=w))
    del d
    torch.cuda.empty_cache()


@pytest.mark.parametrize("k", [2, 3, 4, 5])
def test_full_size_sampled(k):
    _check_full_size(W.config(k), k)


def test_full_size_sampled_mixed_shuffled():
    # the mixed step with its requests in a random order (the chunk is not first)
    _check_full_size(W.config(4, shuffle=True), 4)


# ------------------------------------------------------------- properties

def test_plan_reuse_across_layers_and_determinism():
    wl = W.llama8b_decode(seed=2, R=8)
    d = prepare(wl)
    plan = plan_for(wl, d, -1, min_chunk=64)
    assert ak.ak_plan_info(plan)["split_units"] > 0
    first = run(wl, d, plan)
    again = run(wl, d, plan)
    assert torch.equal(first[0], again[0]) and torch.equal(first[1], again[1])
    for layer in range(3):   # fresh Q per "layer", same plan
        q = torch.empty_like(d["q"])
        R.fill_torch(q, 100 + layer, "q")
        out, lse = run(wl, d, plan, q=q)
        from tests.gpu_harness import compare
        from oracle import workload_run as orun
        qh = R.values_np(100 + layer, "q", np.arange(q.numel()), "bf16").reshape(q.shape)
        ref_o, ref_l = orun.run(wl, q=qh.astype(np.float64))
        eo = float(np.max(np.abs(out.float().cpu().numpy() - ref_o)))
        el = float(np.max(np.abs(lse.cpu().numpy() - ref_l)))
        say(f"  layer {layer}: max|dout|={eo:.3e} max|dlse|={el:.3e}")
        assert eo <= 2e-2 and el <= 1e-3


@pytest.mark.parametrize("kd", ["bf16", "fp8"])
def test_large_scores_raise_the_reference(kd):
    # Queries scaled by 8 (exact in bf16) spread the scores over tens of base-2
    # units, so tiles after the first keep exceeding the running reference by
    # more than the lazy margin: the large-tile fast path's late check takes the
    # tile max, rescales and recomputes, and the decode path raises per block.
    wl = W.custom(seed=31, q_lens=[200, 1, 129, 1], kv_lens=[4000, 2500, 1300, 700], page_size=16,
                  num_qo_heads=16, num_kv_heads=4, head_dim=128, kv_dtype=kd, windows=(-1, 600),
                  name=f"large_scores_{kd}")
    say(f"[parity] large scores, {kd} caches")
    # Error bound: P is rounded to bf16 before the PV product (relative error at
    # most 2^-8 of each weight, so at most 2^-8 max|v| in the output) and the
    # output is rounded to bf16 (at most 2^-8 |out| <= 2^-8 max|v|).  With scores
    # this spread the softmax is peaked and |out| comes close to max|v|, so the
    # fixed 2e-2 of averaged outputs does not apply; max|v| is the largest value
    # the generator's normal table holds (fp8 caches hold scaled codes of it).
    vmax = float(np.abs(R.TABLE_F32).max())
    tol_o = 2.0 ** -7 * vmax * 1.02
    d = prepare(wl)
    from oracle import workload_run as orun
    q = (d["q"].float() * 8.0).to(d["q"].dtype)
    qh = orun.decoded_q(wl) * 8.0
    for window in wl.windows:
        plan = plan_for(wl, d, window)
        assert ak.ak_plan_info(plan)["large_items"] > 0
        out, lse = run(wl, d, plan, q=q)
        ref_o, ref_l = orun.run(wl, window=window, q=qh)
        eo = float(np.max(np.abs(out.float().cpu().numpy() - ref_o)))
        el = float(np.max(np.abs(lse.cpu().numpy() - ref_l)))
        say(f"  window {window}: max|dout|={eo:.3e} max|dlse|={el:.3e}")
        assert eo <= tol_o and el <= 1e-3


@pytest.mark.parametrize("min_chunk,max_splits", [(64, 0), (64, 2), (256, 3)])
def test_forced_splits(min_chunk, max_splits):
    wl = W.llama8b_decode(seed=7, R=6)
    d = prepare(wl)
    plan = plan_for(wl, d, -1, min_chunk=min_chunk, max_splits=max_splits, num_cus=512)
    info = ak.ak_plan_info(plan)
    assert info["split_units"] > 0
    out, lse = run(wl, d, plan)
    check(wl, out, lse, -1)


# ------------------------------------------------------------- edge cases

EDGE = [
    # name, q_lens, kv_lens, B, hq, hkv, D, q_dtype, kv_dtype, causal, windows
    ("one_key", [1, 1, 1], [1, 2, 17], 16, 8, 2, 128, "bf16", "bf16", True, (-1, 0)),
    ("zero_query_rows", [0, 3, 0, 1], [5, 40, 9, 70], 16, 8, 2, 128, "bf16", "bf16", True, (-1, 4)),
    ("page_size_1", [1, 5, 1], [300, 77, 1], 1, 32, 8, 128, "bf16", "bf16", True, (-1, 31)),
    ("page_size_256", [1, 2, 130], [1000, 513, 700], 256, 32, 8, 128, "bf16", "bf16", True, (-1, 100)),
    ("mha_g1", [1, 20, 1], [90, 200, 400], 16, 8, 8, 128, "bf16", "bf16", True, (-1,)),
    ("gqa_g16", [1, 1, 9], [700, 65, 300], 16, 32, 2, 128, "bf16", "bf16", True, (-1, 50)),
    ("head_dim_64", [1, 37, 1], [333, 260, 64], 16, 16, 4, 64, "bf16", "bf16", True, (-1, 20)),
    ("non_causal", [64, 200, 1], [64, 511, 90], 16, 8, 2, 128, "bf16", "bf16", False, (-1,)),
    ("fp8_prefill", [1, 150, 2], [3000, 900, 65], 64, 16, 2, 128, "bf16", "fp8", True, (-1, 300)),
    # fp8 caches on the large-tile path: head_dim 64, token slots (page 1), several
    # 128-token blocks with a ragged tail, non-causal, and a window straddling blocks
    ("fp8_prefill_d64", [37, 1, 300], [333, 64, 700], 16, 16, 4, 64, "bf16", "fp8", True, (-1, 20)),
    ("fp8_prefill_page1", [129, 64, 1], [1000, 64, 300], 1, 32, 8, 128, "bf16", "fp8", True, (-1, 200)),
    ("fp8_noncausal", [64, 200, 1], [64, 511, 90], 16, 8, 2, 128, "bf16", "fp8", False, (-1,)),
    ("fp8_window_straddle", [128, 128], [178, 300], 16, 8, 8, 128, "bf16", "fp8", True, (80, 40, 7)),
    ("fp32_prefill", [1, 70, 3], [40, 100, 200], 16, 8, 2, 64, "f32", "f32", True, (-1, 10)),
    ("fp32_d128", [2, 1], [33, 129], 4, 4, 1, 128, "f32", "f32", True, (-1,)),
    ("multi_row_small", [2, 4, 3], [2000, 1500, 999], 16, 8, 2, 128, "bf16", "bf16", True, (-1, 700)),
    # regression: a decode-shaped tile whose first query row sees nothing in the
    # last KV block while the second row does (its running max must stay finite)
    ("multi_row_tail", [2, 2], [65, 33], 64, 16, 2, 128, "bf16", "bf16", True, (-1, 1)),
    # regression: a prefill tile where the window start (clamped at 0 for early
    # rows) makes some rows of a wave see nothing in a block that others see
    ("window_straddle", [128, 128], [178, 300], 16, 8, 8, 128, "bf16", "bf16", True, (80, 40, 7)),
]


@pytest.mark.parametrize("case", EDGE, ids=[c[0] for c in EDGE])
def test_edge_cases(case):
    name, ql, kl, B, hq, hkv, D, qd, kd, causal, windows = case
    wl = W.custom(seed=len(name) * 31 + sum(kl), q_lens=ql, kv_lens=kl, page_size=B,
                  num_qo_heads=hq, num_kv_heads=hkv, head_dim=D, q_dtype=qd, kv_dtype=kd,
                  causal=causal, windows=windows, name=name)
    say(f"[edge] {name}")
    d = prepare(wl)
    for window in windows:
        for kw in ({}, {"min_chunk": 64, "num_cus": 1024}):
            plan = plan_for(wl, d, window, **kw)
            out, lse = run(wl, d, plan)
            check(wl, out, lse, window)


def test_empty_batch_launches_nothing():
    q = torch.empty(0, 8, 128, dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros(2, 16, 2, 128, dtype=torch.bfloat16, device="cuda")
    idx = torch.zeros(0, dtype=torch.int32, device="cuda")
    plan = ak.ak_plan([0], [0], idx, [], 8, 2, 128, 16)
    out, _ = ak.ak_run(plan, q, kc, kc)
    assert out.shape == q.shape


def test_run_rejects_mismatched_geometry():
    wl = W.custom(seed=9, q_lens=[1, 1], kv_lens=[20, 30], page_size=16, num_qo_heads=8,
                  num_kv_heads=2, head_dim=128)
    d = prepare(wl)
    plan = plan_for(wl, d, -1)
    q16 = torch.zeros(2, 16, 128, dtype=torch.bfloat16, device="cuda")   # more heads than planned
    with pytest.raises(ak.AkError) as e:
        ak.ak_run(plan, q16, d["k_cache"], d["v_cache"])
    assert e.value.status == ak.AK_ERR_SHAPE_MISMATCH
    with pytest.raises(ak.AkError) as e:
        ak.ak_run(plan, d["q"].float(), d["k_cache"], d["v_cache"])
    assert e.value.status == ak.AK_ERR_UNSUPPORTED
    kc8 = d["k_cache"].view(-1)[: d["k_cache"].numel() // 2].view(
        d["k_cache"].shape[0], 8, 2, 128)                                  # wrong page size
    with pytest.raises(ak.AkError) as e:
        ak.ak_run(plan, d["q"], kc8, kc8)
    assert e.value.status == ak.AK_ERR_SHAPE_MISMATCH
    # cache strides the kernels cannot address are refused before any launch
    # (descriptors edited directly: no view of that size is ever built)
    import ctypes
    for dim, stride in ((0, 1 << 30), (1, 1 << 23)):
        dq, dk, dv, do = (ak.tensor_desc(d["q"]), ak.tensor_desc(d["k_cache"]),
                          ak.tensor_desc(d["v_cache"]), ak.tensor_desc(torch.empty_like(d["q"])))
        dk.stride[dim] = stride
        st = ak.lib().ak_run(plan.handle, ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv),
                             ctypes.byref(do), None, None)
        assert st == ak.AK_ERR_UNSUPPORTED and "strides" in ak.ak_last_error()


# ------------------------------------------------------ layouts and splits

@pytest.mark.parametrize("kd", ["bf16", "fp8"])
def test_strided_views(kd):
    # K and V interleaved in one pool [P, B, 2, Hkv, D], q a slice of a fused
    # [T, Hq + 2 Hkv, D] projection, out a slice of a wider buffer, lse strided
    wl = W.custom(seed=17, q_lens=[1, 1, 90, 3], kv_lens=[700, 33, 300, 2100], page_size=16,
                  num_qo_heads=16, num_kv_heads=4, head_dim=128, kv_dtype=kd, windows=(-1, 64),
                  name=f"strided_{kd}")
    say(f"[layout] strided views, {kd} caches")
    d = prepare(wl)
    P, B, H, D = d["k_cache"].shape
    pool = torch.empty(P, B, 2, H, D, dtype=d["k_cache"].dtype, device="cuda")
    pool[:, :, 0] = d["k_cache"]
    pool[:, :, 1] = d["v_cache"]
    kc, vc = pool[:, :, 0], pool[:, :, 1]
    T, Hq = wl.total_q, wl.num_qo_heads
    qkv = torch.empty(T, Hq + 2 * H, D, dtype=d["q"].dtype, device="cuda")
    qkv[:, :Hq] = d["q"]
    q = qkv[:, :Hq]
    assert not q.is_contiguous() and not kc.is_contiguous()
    for window in wl.windows:
        for kw in ({}, {"min_chunk": 64, "num_cus": 1024}):
            plan = plan_for(wl, d, window, **kw)
            wide = torch.full((T, Hq + 4, D), float("nan"), dtype=d["q"].dtype, device="cuda")
            out = wide[:, 2:2 + Hq]
            lse_wide = torch.full((T, 2 * Hq), float("nan"), device="cuda")
            lse = lse_wide[:, ::2]
            ak.ak_run(plan, q, kc, vc, out=out, lse=lse, k_scale=wl.kv_scale, v_scale=wl.kv_scale)
            torch.cuda.synchronize()
            check(wl, out, lse, window)
            # nothing outside the views was written
            assert torch.all(torch.isnan(wide[:, :2].float())) and torch.all(torch.isnan(wide[:, 2 + Hq:].float()))
            assert torch.all(torch.isnan(lse_wide[:, 1::2]))


@pytest.mark.parametrize("kd,D", [("bf16", 128), ("fp8", 128), ("bf16", 64), ("fp8", 64)])
def test_prefill_copies_with_64bit_offsets(kd, D):
    # The prefill kernels form their copy addresses in 32 bits when the pool's
    # page stride, page count and span allow it; a page stride of 2^24 bytes (the
    # caches as views into a wider buffer) takes the 64-bit form instead.
    wl = W.custom(seed=23, q_lens=[90, 1, 130, 70], kv_lens=[300, 40, 700, 70], page_size=64,
                  num_qo_heads=16, num_kv_heads=4, head_dim=D, kv_dtype=kd, windows=(-1, 100),
                  name=f"copy64_{kd}_{D}")
    say(f"[layout] prefill copies with 64-bit offsets, {kd} caches, head_dim {D}")
    d = prepare(wl)
    P, B, H, D = d["k_cache"].shape
    eb = d["k_cache"].element_size()
    sp = (1 << 24) // eb                     # page stride of 2^24 bytes, in elements
    views = []
    for c in (d["k_cache"], d["v_cache"]):
        buf = torch.zeros(P * sp, dtype=c.dtype, device="cuda")
        v = buf.as_strided((P, B, H, D), (sp, H * D, D, 1))
        v.copy_(c)
        views.append(v)
    for window in wl.windows:
        plan = plan_for(wl, d, window)
        assert ak.ak_plan_info(plan)["large_items"] > 0
        out = torch.full_like(d["q"], float("nan"))
        lse = torch.full((wl.total_q, wl.num_qo_heads), float("nan"), device="cuda")
        ak.ak_run(plan, d["q"], views[0], views[1], out=out, lse=lse, k_scale=wl.kv_scale,
                  v_scale=wl.kv_scale)
        torch.cuda.synchronize()
        check(wl, out, lse, window)
        # the same bits as the 32-bit form on the compact caches
        o2, l2 = run(wl, d, plan)
        assert torch.equal(out, o2) and torch.equal(lse, l2)


def test_page_table_span_forces_more_splits():
    # page size 1 and at most 2 splits: a part may not span more than the 1024
    # pages a small tile stages, so the planner cuts more parts than max_splits
    wl = W.custom(seed=23, q_lens=[1, 1, 2], kv_lens=[5000, 3000, 2049], page_size=1,
                  num_qo_heads=8, num_kv_heads=2, head_dim=128, name="span_split")
    say("[splits] page-table span")
    d = prepare(wl)
    plan = plan_for(wl, d, -1, max_splits=2)
    items, _ = ak.ak_plan_export(plan)
    per_unit = {}
    for it in items.tolist():
        per_unit[(it[0], it[1])] = per_unit.get((it[0], it[1]), 0) + 1
        assert it[5] - it[4] <= 1024          # each part within one staged page table
    assert max(per_unit.values()) > 2
    out, lse = run(wl, d, plan)
    check(wl, out, lse, -1)


def test_long_prefill_split_along_kv():
    # one long extend over a long prefix: its few 256-row jobs would set the
    # makespan, so the planner splits them along KV and merges the parts
    wl = W.custom(seed=29, q_lens=[512], kv_lens=[16384], page_size=16, num_qo_heads=32,
                  num_kv_heads=8, head_dim=128, name="long_prefill")
    say("[splits] long prefill, large tiles split along KV")
    d = prepare(wl)
    plan = plan_for(wl, d, -1)
    info = ak.ak_plan_info(plan)
    say(f"  plan {info}")
    assert info["large_items"] > 64 and info["merge_jobs"] > 0
    out, lse = run(wl, d, plan)
    check(wl, out, lse, -1, rows_of=lambda r: _sample_rows(wl, r, k=48))
