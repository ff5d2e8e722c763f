"""Fixed (graph-capturable) plans on the host: capacity bounds and equality
with ordinary plans.

A fixed plan sizes its workspace once from the batch maxima; every batch inside
the documented range must fit it, whatever its mix of decode, extend and
prefill requests, and its work list must be the one an ordinary plan of the
same batch gets (the same planner), so that runs of either are identical.
"""

import numpy as np
import pytest

import paged_kv_attention_store_amd as ak


def _csr(q_lens, kv_lens, B):
    q = np.asarray(q_lens, np.int64)
    L = np.asarray(kv_lens, np.int64)
    pages = -(-L // B)
    qo = np.concatenate([[0], np.cumsum(q)]).astype(np.int32)
    kv = np.concatenate([[0], np.cumsum(pages)]).astype(np.int32)
    last = np.where(pages > 0, L - (pages - 1) * B, 0).astype(np.int32)
    return qo, kv, last


def _batch(rng, kind, max_batch, max_tokens, G, Hkv, B, lmax, kv_budget, page_budget=None):
    """Query and KV lengths of one batch of the given kind inside the maxima."""
    small_n = max(1, 16 // G)                      # most tokens a small unit can hold
    if kind == "decode":
        R = max_batch if rng.random() < 0.5 else int(rng.integers(1, max_batch + 1))
        R = min(R, max_tokens)
        n = np.ones(R, np.int64)
    elif kind == "small_units":                    # every request just fits a small tile
        R = min(max_batch, max_tokens // small_n)
        n = np.full(R, small_n, np.int64)
    elif kind == "many_jobs":                      # as many large jobs as the tokens allow
        per = small_n + 1
        R = max(1, min(max_batch, max_tokens // per))
        n = np.full(R, per, np.int64)
    elif kind == "one_prefill":
        R = 1
        n = np.array([max_tokens], np.int64)
    else:                                          # random mix
        R = int(rng.integers(1, max_batch + 1))
        cuts = np.sort(rng.integers(0, max_tokens + 1, size=R - 1))
        n = np.diff(np.concatenate([[0], cuts, [int(rng.integers(R, max_tokens + 1))]]))
        n = np.maximum(n, 0)
        if n.sum() > max_tokens:
            n[:] = 1
    R = len(n)
    if R == 0:
        return n, n
    # KV lengths: long where the budget allows, never below n (causal)
    cap = max(1, min(lmax, kv_budget // (Hkv * R)))
    L = np.maximum(n, rng.integers(1, cap + 1, size=R))
    if rng.random() < 0.5:
        L = np.maximum(n, np.full(R, cap))
    while Hkv * L.sum() > kv_budget:
        L = np.maximum(n, L // 2)
    if page_budget is not None:
        n, L = n[:page_budget], L[:page_budget]     # every request holds a page
        while (-(-L // B)).sum() > page_budget and L.max() > 1:
            L = np.maximum(np.minimum(n, 1), L // 2)
            n = np.minimum(n, L)
    return n, L


def _live(items):
    """The work items with rows (padding items have none), in a canonical order."""
    live = items[items[:, 3] > 0]
    return live[np.lexsort(live.T[::-1])]


CASES = [
    # max_batch, max_tokens, Hq, Hkv, B, num_cus, max_splits
    (64, 64, 32, 8, 16, 256, 0),
    (256, 2304, 32, 8, 64, 256, 0),
    (8, 16384, 32, 8, 16, 256, 0),
    (128, 512, 64, 8, 16, 80, 16),
    (32, 4096, 8, 8, 8, 256, 4),
    (16, 1024, 16, 1, 32, 304, 0),
    (512, 512, 16, 16, 16, 256, 2),
]


@pytest.mark.parametrize("pages", [None, 3000, 200], ids=["pages_any", "pages_3000", "pages_200"])
@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_fixed_capacity_holds_every_batch(case, pages):
    max_batch, max_tokens, Hq, Hkv, B, cus, S = case
    G = Hq // Hkv
    splits = S or 64
    lmax = splits * (1022 * B - 128)
    kv_budget = 6 * cus * 4096
    plan = ak.ak_plan_fixed(max_batch, max_tokens, None, Hq, Hkv, 128, B, num_cus=cus,
                            max_splits=S, host_only=True, max_pages=pages or (1 << 30))
    info = plan.info()
    rng = np.random.default_rng(max_batch + max_tokens + B)
    peak = dict.fromkeys(["small_items", "large_items", "merge_jobs", "partial_rows"], 0)
    for trial in range(60):
        kind = ["decode", "small_units", "many_jobs", "one_prefill", "mix"][trial % 5]
        n, L = _batch(rng, kind, max_batch, max_tokens, G, Hkv, B, lmax, kv_budget, pages)
        qo, kv, last = _csr(n, L, B)
        ak.ak_plan_update(plan, qo, kv, last)        # raises if the batch does not fit
        got = plan.info()
        for k in peak:
            peak[k] = max(peak[k], got[k])
        assert got["small_items"] <= info["cap_small_items"]
        assert got["large_items"] <= info["cap_large_items"]
        assert got["merge_jobs"] <= info["cap_merge_jobs"]
        assert got["partial_rows"] <= info["cap_partial_rows"]
        # the same work list as an ordinary plan of this batch
        ref = ak.ak_plan(qo, kv, None, last, Hq, Hkv, 128, B, num_cus=cus, max_splits=S,
                         host_only=True)
        # (an ordinary plan of few prefill units groups their segments by die,
        # which reorders the large items and pads them with empty ones; a fixed
        # plan keeps longest-first order, so the live items are compared as a set)
        a_items, a_lens = ak.ak_plan_export(plan)
        b_items, b_lens = ak.ak_plan_export(ref)
        assert np.array_equal(_live(a_items), _live(b_items)) and np.array_equal(a_lens, b_lens)
        same = lambda d: {k: v for k, v in d.items()
                          if not k.startswith("cap_") and k not in ("items", "large_items")}
        assert same(got) == same(ref.info())
        assert len(_live(a_items)) == len(_live(b_items))
    # the batches exercised the bounds (not a vacuous pass)
    assert peak["small_items"] > 0 or peak["large_items"] > 0


def test_fixed_plan_rejects_batches_over_capacity():
    plan = ak.ak_plan_fixed(4, 32, None, 32, 8, 128, 16, host_only=True, max_pages=100)
    qo, kv, last = _csr([1] * 5, [20] * 5, 16)
    with pytest.raises(ak.AkError) as e:
        ak.ak_plan_update(plan, qo, kv, last)       # 5 requests > 4
    assert e.value.status == ak.AK_ERR_SHAPE_MISMATCH
    qo, kv, last = _csr([30, 3], [40, 40], 16)
    with pytest.raises(ak.AkError) as e:
        ak.ak_plan_update(plan, qo, kv, last)       # 33 tokens > 32
    assert e.value.status == ak.AK_ERR_SHAPE_MISMATCH
    qo, kv, last = _csr([1, 1], [1600, 16], 16)
    with pytest.raises(ak.AkError) as e:
        ak.ak_plan_update(plan, qo, kv, last)       # 101 pages > 100
    assert e.value.status == ak.AK_ERR_SHAPE_MISMATCH
    # a failed update leaves the previous batch in place
    qo, kv, last = _csr([1, 2], [40, 50], 16)
    ak.ak_plan_update(plan, qo, kv, last)
    before = ak.ak_plan_export(plan)
    with pytest.raises(ak.AkError):
        ak.ak_plan_update(plan, [0, 1], [0, 2], [17])   # last_page_len > page_size
    after = ak.ak_plan_export(plan)
    assert np.array_equal(before[0], after[0]) and plan.info()["batch_size"] == 2
    # an ordinary plan cannot be updated; causal geometry errors surface at creation
    ordinary = ak.ak_plan(qo, kv, None, last, 32, 8, 128, 16, host_only=True)
    with pytest.raises(ak.AkError) as e:
        ak.ak_plan_update(ordinary, qo, kv, last)
    assert e.value.status == ak.AK_ERR_INVALID_ARG
    with pytest.raises(ak.AkError) as e:
        ak.ak_plan_fixed(4, 32, None, 32, 8, 96, 16, host_only=True, max_pages=10)
    assert e.value.status == ak.AK_ERR_UNSUPPORTED


def test_fixed_plan_empty_batch_and_shrinking_batches():
    plan = ak.ak_plan_fixed(16, 64, None, 32, 8, 128, 16, host_only=True, max_pages=4096)
    ak.ak_plan_update(plan, [0], [0], np.zeros(0, np.int32))
    assert plan.info()["items"] == 0 and plan.info()["batch_size"] == 0
    for R in (16, 3, 9, 1):
        qo, kv, last = _csr([1] * R, [3000] * R, 16)
        ak.ak_plan_update(plan, qo, kv, last)
        assert plan.info()["batch_size"] == R


@pytest.mark.parametrize("case", CASES[:4], ids=[f"c{i}" for i in range(4)])
def test_fixed_capacity_with_query_length_bound(case):
    max_batch, max_tokens, Hq, Hkv, B, cus, S = case
    G = Hq // Hkv
    for qlen in (1, 16 // G + 1, 300):
        plan = ak.ak_plan_fixed(max_batch, max_tokens, None, Hq, Hkv, 128, B, num_cus=cus,
                                max_splits=S, host_only=True, max_pages=1 << 30,
                                max_query_len=qlen)
        info = plan.info()
        if qlen * G <= 16:
            assert info["cap_large_items"] == 0          # pure decode: no large-tile launch
        rng = np.random.default_rng(qlen)
        for trial in range(40):
            kind = ["decode", "small_units", "many_jobs", "one_prefill", "mix"][trial % 5]
            n, L = _batch(rng, kind, max_batch, max_tokens, G, Hkv, B, (S or 64) * 1000,
                          6 * cus * 4096)
            n = np.minimum(n, qlen)
            L = np.maximum(L, n)
            qo, kv, last = _csr(n, L, B)
            ak.ak_plan_update(plan, qo, kv, last)
            got = plan.info()
            for k in ("small_items", "large_items", "merge_jobs", "partial_rows"):
                cap = "cap_" + k
                assert got[k] <= info[cap]
    # a request longer than max_query_len is refused
    plan = ak.ak_plan_fixed(8, 64, None, 32, 8, 128, 16, host_only=True, max_pages=100,
                            max_query_len=1)
    qo, kv, last = _csr([1, 2], [40, 40], 16)
    with pytest.raises(ak.AkError) as e:
        ak.ak_plan_update(plan, qo, kv, last)
    assert e.value.status == ak.AK_ERR_SHAPE_MISMATCH
