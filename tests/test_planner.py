"""Host planner checks through the C ABI with host-only plans (no GPU):
validation status codes, lengths, and that the work list covers every visible
(query token, query head, key) triple exactly once."""

import numpy as np
import pytest

import paged_kv_attention_store_amd as ak
from oracle import metadata as M
from synth import workloads as W


def host_plan(qo, kv, last, hq=8, hkv=2, d=128, B=16, causal=True, window=-1, **kw):
    return ak.ak_plan(qo, kv, None, last, hq, hkv, d, B, causal=causal, window=window,
                      host_only=True, **kw)


def _status(fn):
    with pytest.raises(ak.AkError) as e:
        fn()
    return e.value.status


# ------------------------------------------------------------- validation

def test_bad_indptr():
    assert _status(lambda: host_plan([1, 2], [0, 1], [1])) == ak.AK_ERR_BAD_INDPTR
    assert _status(lambda: host_plan([0, 2, 1], [0, 1, 2], [1, 1])) == ak.AK_ERR_BAD_INDPTR
    assert _status(lambda: host_plan([0, 1, 2], [0, 2, 1], [1, 1])) == ak.AK_ERR_BAD_INDPTR


def test_bad_lengths():
    assert _status(lambda: host_plan([0, 1], [0, 1], [0])) == ak.AK_ERR_BAD_LENGTHS
    assert _status(lambda: host_plan([0, 1], [0, 1], [17])) == ak.AK_ERR_BAD_LENGTHS
    # 5 queries but only 4 keys
    assert _status(lambda: host_plan([0, 5], [0, 1], [4])) == ak.AK_ERR_BAD_LENGTHS
    # queries on a request without pages
    assert _status(lambda: host_plan([0, 1], [0, 0], [1])) == ak.AK_ERR_BAD_LENGTHS


def test_invalid_and_unsupported_geometry():
    ok = ([0, 1], [0, 1], [3])
    assert _status(lambda: host_plan(*ok, hq=6, hkv=4)) == ak.AK_ERR_INVALID_ARG
    assert _status(lambda: host_plan(*ok, hq=24, hkv=1)) == ak.AK_ERR_UNSUPPORTED   # G = 24
    assert _status(lambda: host_plan(*ok, d=96)) == ak.AK_ERR_UNSUPPORTED
    assert _status(lambda: host_plan(*ok, B=12)) == ak.AK_ERR_UNSUPPORTED
    assert _status(lambda: host_plan(*ok, B=512)) == ak.AK_ERR_UNSUPPORTED
    assert _status(lambda: host_plan(*ok, causal=False, window=8)) == ak.AK_ERR_UNSUPPORTED
    assert _status(lambda: host_plan(*ok, window=-2)) == ak.AK_ERR_INVALID_ARG


def test_error_text_is_set():
    with pytest.raises(ak.AkError):
        host_plan([0, 5], [0, 1], [4])
    assert "queries" in ak.ak_last_error()


def test_empty_batch_and_zero_query_requests():
    p = host_plan([0], [0], [])
    assert ak.ak_plan_info(p)["items"] == 0
    p = host_plan([0, 0, 0], [0, 2, 3], [5, 16])
    info = ak.ak_plan_info(p)
    assert info["items"] == 0 and info["total_q"] == 0


def test_host_only_plan_cannot_run():
    p = host_plan([0, 1], [0, 1], [3])
    with pytest.raises(ak.AkError) as e:
        ak.ak_run(p, *([_FakeTensor()] * 3), out=_FakeTensor())
    assert e.value.status == ak.AK_ERR_INVALID_ARG


class _FakeTensor:
    """Enough of a tensor for the descriptor code; never dereferenced."""
    import torch as _t
    dtype = _t.bfloat16
    shape = (1, 8, 128)

    def dim(self):
        return 3

    def numel(self):
        return 1

    def data_ptr(self):
        return 16

    def stride(self, i=None):
        st = (1024, 128, 1)
        return st if i is None else st[i]


# --------------------------------------------------------------- coverage

def _row_ranges(L, n, G, causal, window, rows):
    j = rows // G
    qpos = L - n + j
    hi = qpos + 1 if causal else np.full_like(qpos, L)
    lo = np.maximum(0, qpos - window) if window >= 0 else np.zeros_like(qpos)
    return lo, hi


def check_coverage(qo, kv, last, B, hq, hkv, causal, window, **kw):
    G = hq // hkv
    p = host_plan(qo, kv, last, hq=hq, hkv=hkv, B=B, causal=causal, window=window, **kw)
    items, lens = ak.ak_plan_export(p)
    Ls = M.kv_lengths(kv, last, B)
    ns = M.q_lengths(qo)
    assert lens.tolist() == Ls.tolist()
    info = ak.ak_plan_info(p)
    assert info["total_q"] == int(qo[-1])
    # per (request, kv head): count of coverage of each (row, key)
    cover = {}
    partial_rows = set()
    for r, hk, row0, nrows, kb, ke, pbase, kind in items.tolist():
        if nrows == 0:
            # an empty item (padding between the dies' lists of large segments)
            assert kind == 1 and kb == ke == 0 and pbase == -1
            continue
        assert 0 <= kb <= ke <= Ls[r]
        assert kind == (0 if ns[r] * G <= 16 else 1)
        key = (r, hk)
        if key not in cover:
            cover[key] = np.zeros((ns[r] * G, Ls[r]), dtype=np.int32)
        cover[key][row0:row0 + nrows, kb:ke] += 1
        if pbase >= 0:
            rows = set(range(pbase, pbase + nrows))
            assert not rows & partial_rows
            partial_rows |= rows
    assert len(partial_rows) == info["partial_rows"]
    for r in range(len(ns)):
        if ns[r] == 0:
            continue
        for hk in range(hkv):
            c = cover[(r, hk)]
            rows = np.arange(ns[r] * G)
            lo, hi = _row_ranges(Ls[r], ns[r], G, causal, window, rows)
            t = np.arange(Ls[r])[None, :]
            vis = (t >= lo[:, None]) & (t < hi[:, None])
            # every visible key covered exactly once; invisible keys may be swept
            # by a tile's range (masked in the kernel) but never twice
            assert np.all(c[vis] == 1), (r, hk)
            assert np.all(c <= 1)
    return p, items


def test_coverage_worked_example_shapes():
    # vLLM worked example geometry: one decode + two extends
    qo = [0, 1, 5, 8]
    kv = [0, 8, 9, 12]
    last = [16, 4, 3]
    check_coverage(qo, kv, last, 16, 8, 2, True, -1)
    check_coverage(qo, kv, last, 16, 8, 2, True, 5)


@pytest.mark.parametrize("seed", range(12))
def test_coverage_random_batches(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.choice([1, 2, 16, 64]))
    G = int(rng.choice([1, 2, 4, 8]))
    hkv = int(rng.choice([1, 2]))
    R = int(rng.integers(1, 7))
    Ls = rng.integers(1, 700, size=R)
    ns = np.array([int(rng.integers(0, min(L, 80) + 1)) if rng.random() < 0.5 else min(1, L)
                   for L in Ls])
    pages = -(-Ls // B)
    kv = np.concatenate([[0], np.cumsum(pages)])
    qo = np.concatenate([[0], np.cumsum(ns)])
    last = Ls - (pages - 1) * B
    window = int(rng.choice([-1, 0, 3, 50, 1000]))
    causal = True if window >= 0 else bool(rng.random() < 0.7)
    check_coverage(qo, kv, last, B, G * hkv, hkv, causal, window,
                   min_chunk=64, num_cus=int(rng.choice([4, 64, 256])))


@pytest.mark.parametrize("k", [2, 4, 5])
def test_split_partition_of_full_configs(k):
    wl = W.config(k)
    for window in wl.windows:
        p = host_plan(wl.qo_indptr, wl.kv_indptr, wl.last_page_len, hq=wl.num_qo_heads,
                      hkv=wl.num_kv_heads, B=wl.page_size, causal=wl.causal, window=window)
        info = ak.ak_plan_info(p)
        items, lens = ak.ak_plan_export(p)
        assert lens.tolist() == wl.kv_lens.tolist()
        small = items[items[:, 7] == 0]
        # every split KV range is at most 4096 tokens and splits tile their unit
        assert np.all(small[:, 5] - small[:, 4] <= 4096 + 64)
        if k == 5:
            assert info["split_units"] == 64 and info["small_items"] >= 256
        # the workspace holds far fewer bytes than the KV it summarises
        assert info["partial_rows"] * (wl.head_dim + 1) * 4 < 0.02 * wl.kv_lens.sum() * \
            wl.num_kv_heads * wl.head_dim * 2 * (1 if wl.kv_dtype == "fp8" else 2)


def test_over_planning_trap_is_a_hard_check():
    # a plan built for 8 query heads cannot run a 16-head q: checked in ak_run
    # (shape mismatch) -- here: the plan records its head geometry
    p = host_plan([0, 1], [0, 1], [3], hq=8, hkv=2)
    assert p.num_qo_heads == 8


# ------------------------------------------------------- large-tile order

# ------------------------------------------------------- decode split

def _small(p):
    items, _ = ak.ak_plan_export(p)
    info = ak.ak_plan_info(p)
    return items[:info["small_items"]], info


@pytest.mark.parametrize("k", [2, 4, 5])
@pytest.mark.parametrize("num_cus", [64, 256])
def test_decode_parts_longest_first_even_and_bounded(k, num_cus):
    # decode items launch longest KV range first; a unit's parts tile its visible
    # range without gaps, none empty, sizes within two 64-token grid steps of each
    # other (the first part is shorter by the unit's offset from the grid); the
    # count respects the fixed-plan bound units + 4 * 6 * num_cus where that bound
    # is stated (decode KV <= 6 * num_cus * 4096 tokens over the KV heads), and
    # units + KV / 1024 (parts of at least a quarter of the 4096-token chunk cap)
    # beyond it
    wl = W.config(k)
    for w in wl.windows:
        p = host_plan(wl.qo_indptr, wl.kv_indptr, wl.last_page_len, hq=wl.num_qo_heads,
                      hkv=wl.num_kv_heads, B=wl.page_size, causal=True, window=w, num_cus=num_cus)
        small, info = _small(p)
        ln = small[:, 5] - small[:, 4]
        assert np.all(ln > 0) and np.all(np.diff(ln) <= 0)
        units = {}
        for it in small:
            units.setdefault((int(it[0]), int(it[1])), []).append((int(it[4]), int(it[5])))
        for (r, hk), parts in units.items():
            parts.sort()
            assert all(parts[i][1] == parts[i + 1][0] for i in range(len(parts) - 1))
            L, n = int(wl.kv_lens[r]), int(wl.q_lens[r])
            hi = L if n > 0 else 0
            lo = 0 if w < 0 else max(0, L - n - w)
            assert parts[0][0] == lo and parts[-1][1] == hi
            sizes = [b - a for a, b in parts]
            assert max(sizes) - min(sizes) <= 128, (r, hk, sizes)
        kv = sum(b - a for parts in units.values() for a, b in parts)
        if kv <= 6 * num_cus * 4096:
            assert len(small) <= len(units) + 4 * 6 * num_cus
        else:
            assert len(small) <= len(units) + -(-kv // 1024)


def _large(p):
    items, _ = ak.ak_plan_export(p)
    info = ak.ak_plan_info(p)
    return items[info["small_items"]:], info


def _cost(large):
    return np.ceil((large[:, 5] - large[:, 4]) / 32.0)


XCDS = 8   # dies of the chip: workgroup x runs on die x mod 8


def _die_lists(large):
    """The live large items each die runs, in dispatch order."""
    out = []
    for d in range(XCDS):
        sub = large[d::XCDS]
        out.append(sub[sub[:, 3] > 0])
    return out


def test_large_tiles_longest_first_without_splits():
    # many jobs against 256 compute units: no job exceeds the per-unit share, so
    # nothing is split; the dispatch order is longest KV range first
    wl = W.config(3)
    p = host_plan(wl.qo_indptr, wl.kv_indptr, wl.last_page_len, hq=wl.num_qo_heads,
                  hkv=wl.num_kv_heads, B=wl.page_size, causal=True, window=-1, num_cus=256)
    large, info = _large(p)
    assert len(large) > 256 and np.all(large[:, 6] == -1) and info["merge_jobs"] == 0
    c = _cost(large)
    assert np.all(np.diff(c) <= 0)


@pytest.mark.parametrize("seed", range(8))
def test_large_split_of_few_long_jobs(seed):
    # few long jobs on many compute units: the longest are split along KV; the
    # cover stays exact and every split row gets one merge job over its parts
    rng = np.random.default_rng(100 + seed)
    R = int(rng.integers(1, 4))
    Ls = rng.integers(3000, 9000, size=R)
    ns = np.array([int(rng.integers(17, 300)) for _ in Ls])
    B = 16
    pages = -(-Ls // B)
    kv = np.concatenate([[0], np.cumsum(pages)])
    qo = np.concatenate([[0], np.cumsum(ns)])
    last = Ls - (pages - 1) * B
    P = int(rng.choice([16, 64, 256]))
    p, _ = check_coverage(qo, kv, last, B, 8, 2, True, -1, num_cus=P)
    large, info = _large(p)
    # few units: grouped by die, each die's list longest first
    for lst in _die_lists(large):
        assert np.all(np.diff(_cost(lst)) <= 0)
    large = large[large[:, 3] > 0]
    split = large[large[:, 6] >= 0]
    assert len(split) > 0
    # parts of one job share (request, head, rows) and tile its KV range
    keys = {tuple(x) for x in split[:, :4].tolist()}
    n_merge = 0
    for key in keys:
        parts = split[np.all(split[:, :4] == np.array(key), axis=1)]
        assert len(parts) >= 2
        n_merge += key[3]
    assert info["small_items"] == 0 and n_merge == info["merge_jobs"]


def test_few_units_grouped_by_die():
    # one 2048-token chunk over a 6144-token prefix, 8 KV heads: 8 units of 32
    # segments.  Each unit's segments read the same K/V rows, so all of them run on
    # one die (one L2); the dies' lists are interleaved in dispatch order.
    qo = np.array([0, 2048])
    L = 8192
    B = 64
    kv = np.array([0, L // B])
    last = np.array([B])
    p, _ = check_coverage(qo, kv, last, B, 32, 8, True, -1, num_cus=256)
    large, info = _large(p)
    lists = _die_lists(large)
    for d, lst in enumerate(lists):
        assert len(lst) == 32
        assert len({(r, hk) for r, hk in lst[:, :2].tolist()}) == 1
        assert np.all(np.diff(_cost(lst)) <= 0)
    assert len({tuple(lst[0, :2]) for lst in lists}) == 8
    # many units (the ragged prefill batch): no grouping, longest first overall
    wl = W.config(3)
    p = host_plan(wl.qo_indptr, wl.kv_indptr, wl.last_page_len, hq=wl.num_qo_heads,
                  hkv=wl.num_kv_heads, B=wl.page_size, causal=True, window=-1, num_cus=256)
    large, _ = _large(p)
    assert np.all(large[:, 3] > 0) and np.all(np.diff(_cost(large)) <= 0)


# ------------------------------------------------------- non-causal segments

def test_noncausal_allows_more_queries_than_keys():
    # causal = 0: every key is visible, positions do not matter, so n_r > L_r is a
    # valid request (the prefix segment of a two-segment extend); L_r = 0 is the
    # empty state.  With causal = 1 the same batch is rejected.
    qo, kv, last = [0, 5, 45, 48], [0, 1, 1, 5], [3, 0, 16]
    assert _status(lambda: host_plan(qo, kv, last, causal=True)) == ak.AK_ERR_BAD_LENGTHS
    p, items = check_coverage(np.array(qo), np.array(kv), np.array(last), 16, 8, 2, False, -1)
    # the request without pages is still planned (its rows get the empty state)
    assert set(items[:, 0].tolist()) == {0, 1, 2}
    assert np.all(items[items[:, 0] == 1][:, 4:6] == 0)


# ------------------------------------------------------- host threads

def test_concurrent_planning_from_threads():
    # plans made from eight host threads at once (the calls release the GIL) equal
    # the ones made alone, and each thread's error message is its own
    import threading
    cases = []
    for k in (1, 2, 3, 4):
        wl = W.config(k)
        cases.append((wl.qo_indptr, wl.kv_indptr, wl.last_page_len, wl.num_qo_heads,
                      wl.num_kv_heads, wl.head_dim, wl.page_size))
    ref = []
    for qo, kv, last, hq, hkv, d, B in cases:
        items, lens = ak.ak_plan_export(host_plan(qo, kv, last, hq=hq, hkv=hkv, d=d, B=B))
        ref.append((items.copy(), lens.copy()))
    errors = []

    def worker(tid):
        try:
            for it in range(12):
                c = (tid + it) % len(cases)
                qo, kv, last, hq, hkv, d, B = cases[c]
                if it % 3 == 2:   # a bad request of this thread's own making
                    bad = np.array(last, dtype=np.int32).copy()
                    bad[0] = B + 1 + tid
                    try:
                        host_plan(qo, kv, bad, hq=hq, hkv=hkv, d=d, B=B)
                        errors.append((tid, "accepted a bad last_page_len"))
                    except ak.AkError as e:
                        if e.status != ak.AK_ERR_BAD_LENGTHS or f"= {B + 1 + tid} " not in str(e):
                            errors.append((tid, str(e)))
                    continue
                items, lens = ak.ak_plan_export(host_plan(qo, kv, last, hq=hq, hkv=hkv, d=d, B=B))
                if not (np.array_equal(items, ref[c][0]) and np.array_equal(lens, ref[c][1])):
                    errors.append((tid, f"work list of case {c} differs"))
        except Exception as e:   # noqa: BLE001 - reported below
            errors.append((tid, repr(e)))

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors[:4]
