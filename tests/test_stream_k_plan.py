"""The stream-K decode partition (AK_PLAN_STREAM_K) on the host, through the C
ABI with host-only plans: the decode units' visible KV ranges, laid end to end
in unit order, are cut into equal contiguous shares (four per compute unit); each
share's pieces are consecutive items of one workgroup; every visible (row, key)
is covered exactly once; a unit cut into several pieces gets partial rows and one
merge job per row; pieces fit a small tile's 1024-entry page table."""

import numpy as np
import pytest

import paged_kv_attention_store_amd as ak
from synth import workloads as W
from tests.test_planner import check_coverage, host_plan

SHARES_PER_CU = 4
ALIGN = 64


def _units(items):
    """Small items grouped by unit (request, KV head), in item order."""
    units = {}
    for it in items.tolist():
        units.setdefault((it[0], it[1]), []).append(it)
    return units


def _check_stream_k(qo, kv, last, B, hq, hkv, window, num_cus, causal=True):
    p, items = check_coverage(qo, kv, last, B, hq, hkv, causal, window, stream_k=True,
                              num_cus=num_cus)
    info = ak.ak_plan_info(p)
    wg = ak.ak_plan_workgroups(p)
    small = items[:info["small_items"]]
    P = SHARES_PER_CU * num_cus
    if info["small_items"] == 0:
        return p, small, wg
    assert info["stream_k_workgroups"] == P and len(wg) == P + 1
    assert wg[0] == 0 and wg[-1] == len(small) and np.all(np.diff(wg) >= 0)
    # pieces follow the flattened order: within a unit each starts where the last
    # ended, and units follow each other whole
    for i in range(len(small) - 1):
        a, b = small[i], small[i + 1]
        if (a[0], a[1]) == (b[0], b[1]):
            assert a[5] == b[4]
    # the shares: every workgroup but the last holds at most share + ALIGN tokens
    # (cuts sit on the 64-token grid of each unit), the whole is covered
    ln = small[:, 5] - small[:, 4]
    total = int(ln.sum())
    per = -(-max(total, 1) // P)                         # ceil(total / P)
    share = max(ALIGN, -(-per // ALIGN) * ALIGN)         # rounded up to the grid
    per_wg = np.array([ln[wg[g]:wg[g + 1]].sum() for g in range(P)])
    assert np.all(per_wg[:-1] <= share + ALIGN), (per_wg.max(), share)
    # every piece fits the small tile's page table
    span = (small[:, 5] - 1) // B - small[:, 4] // B + 1
    assert np.all(span[ln > 0] <= 1024)
    # units in one piece write their output directly; the others have partial rows
    # (one per piece and row) and one merge job per row counting their pieces
    small_merges = 0
    for key, its in _units(small).items():
        if len(its) == 1:
            assert its[0][6] == -1
        else:
            assert all(x[6] >= 0 for x in its)
            bases = sorted(x[6] for x in its)
            rows = its[0][3]
            assert bases == [bases[0] + k * rows for k in range(len(its))]
            small_merges += rows
    assert small_merges <= info["merge_jobs"]
    if info["large_items"] == 0:
        assert small_merges == info["merge_jobs"]
    return p, small, wg


@pytest.mark.parametrize("k", [2, 4, 5])
@pytest.mark.parametrize("num_cus", [64, 256])
def test_stream_k_partition_of_full_configs(k, num_cus):
    wl = W.config(k)
    for w in wl.windows:
        _check_stream_k(wl.qo_indptr, wl.kv_indptr, wl.last_page_len, wl.page_size,
                        wl.num_qo_heads, wl.num_kv_heads, w, num_cus)


def test_stream_k_long_decode_is_equal_pieces():
    # 8 x 131072 tokens over 8 KV heads on 256 compute units: 1024 shares of 8192
    # tokens, each exactly one piece, 16 per unit
    wl = W.config(5)
    p, small, wg = _check_stream_k(wl.qo_indptr, wl.kv_indptr, wl.last_page_len, wl.page_size,
                                   wl.num_qo_heads, wl.num_kv_heads, -1, 256)
    assert len(small) == 1024 and np.all(small[:, 5] - small[:, 4] == 8192)
    assert np.all(np.diff(wg) == 1)


@pytest.mark.parametrize("seed", range(10))
def test_stream_k_random_batches(seed):
    rng = np.random.default_rng(500 + seed)
    B = int(rng.choice([1, 2, 16, 64]))
    G = int(rng.choice([1, 2, 4, 8, 16]))
    hkv = int(rng.choice([1, 2, 8]))
    R = int(rng.integers(1, 40))
    Ls = rng.integers(1, 6000, size=R)
    ns = np.array([min(int(rng.choice([0, 1, 1, 1, 2])), int(L)) for L in Ls])
    ns = np.minimum(ns, 16 // G if G <= 16 else 1)
    pages = -(-Ls // B)
    kv = np.concatenate([[0], np.cumsum(pages)])
    qo = np.concatenate([[0], np.cumsum(ns)])
    last = Ls - (pages - 1) * B
    window = int(rng.choice([-1, 0, 100, 3000]))
    _check_stream_k(qo, kv, last, B, G * hkv, hkv, window, int(rng.choice([1, 4, 64, 256])))


def test_stream_k_tiny_pages_are_cut_to_the_page_table():
    # page size 1: no piece may span more than the 1024 staged page ids
    qo, kv, last = [0, 1, 2, 4], [0, 5000, 8000, 10049], [1, 1, 1]
    p, small, _ = _check_stream_k(np.array(qo), np.array(kv), np.array(last), 1, 8, 2, -1, 1)
    assert np.max(small[:, 5] - small[:, 4]) <= 1022


def test_stream_k_with_large_tiles_and_merge_in_kernel():
    # the mixed step: the chunk stays on large tiles, decode units go stream-K,
    # also with the in-kernel merge; the cover stays exact
    wl = W.config(4)
    p = host_plan(wl.qo_indptr, wl.kv_indptr, wl.last_page_len, hq=32, hkv=8, B=64,
                  stream_k=True, merge_in_kernel=True)
    info = ak.ak_plan_info(p)
    assert info["large_items"] > 0 and info["stream_k_workgroups"] == 4 * 256
    check_coverage(wl.qo_indptr, wl.kv_indptr, wl.last_page_len, 64, 32, 8, True, -1,
                   stream_k=True, merge_in_kernel=True)


def test_plain_plans_have_no_workgroup_table():
    p = host_plan([0, 1], [0, 1], [3])
    assert ak.ak_plan_info(p)["stream_k_workgroups"] == 0 and len(ak.ak_plan_workgroups(p)) == 0


def test_fixed_plans_refuse_stream_k():
    with pytest.raises(ak.AkError) as e:
        ak.ak_plan_fixed(8, 8, None, 8, 2, 128, 16, host_only=True, max_pages=64, stream_k=True)
    assert e.value.status == ak.AK_ERR_UNSUPPORTED
