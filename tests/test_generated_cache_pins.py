"""Pins of the oracle's lazily generated KV pools and of the input generator.

Every parity test builds its expected cache through `oracle.workload_run.
GeneratedCache`: the big pools are never held whole, so the code of a slot is
produced on demand (the generated pool value encoded with the oracle's codec)
unless the step's store overwrote it.  Here that lazy view is checked, on pools
small enough to hold whole, against the plain store-then-read of
`oracle.attention.Cache` + `store_kv` (the write rule of the [vLLM backend]
page's "Write the KV first": every non-padding token lands at its slot, in
order), for every cache dtype, with padding slots, slots written twice in one
store and slots overwritten by a second store.

The generator itself (synth.rng) is pinned against its published definition
(Thomas Mueller's 32-bit integer hash, evaluated here in pure Python integers on
a handful of counters, including counters above 2^32) and its host (NumPy) and
device-side (torch) fills are compared bit for bit on the CPU.
"""

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import workload_run as orun
from synth import rng as R
from synth import workloads as W

DTYPES = [("f32", "f32"), ("bf16", "bf16"), ("bf16", "fp8"), ("f32", "fp8"), ("f32", "bf16")]


def _whole_cache(wl, which):
    """The pool held whole: generated values at every slot, encoded."""
    P, B, H, D = wl.num_pages, wl.page_size, wl.num_kv_heads, wl.head_dim
    vals = W.pool_values(wl, which, np.arange(P * B))
    return A.Cache(A.encode(vals, wl.kv_dtype, wl.kv_scale).reshape(P, B, H, D), wl.kv_dtype,
                   wl.kv_scale)


def _stores(wl, rng):
    """Two stores: the workload's own slots with padding (-1) mixed in and one
    slot written twice, then a second store over some of the same slots."""
    base = wl.slot_mapping.copy()
    pad = rng.random(len(base)) < 0.2
    s1 = np.where(pad, -1, base)
    s1 = np.concatenate([s1, [base[0], -7]])              # slot base[0] written twice
    n1 = len(s1)
    v1 = rng.standard_normal((n1, wl.num_kv_heads, wl.head_dim)).astype(np.float32)
    s2 = rng.choice(base, size=max(1, len(base) // 3), replace=False)
    s2 = np.concatenate([s2, [-1]])
    v2 = (3.0 * rng.standard_normal((len(s2), wl.num_kv_heads, wl.head_dim))).astype(np.float32)
    return [(v1, s1), (v2, s2)]


@pytest.mark.parametrize("piece", [8192, 7])
@pytest.mark.parametrize("qd,kd", DTYPES, ids=[f"{a}-{b}" for a, b in DTYPES])
def test_generated_cache_equals_whole_pool_store(qd, kd, piece, monkeypatch):
    # piece = 7: slots generated in many pieces on several threads
    monkeypatch.setattr(orun.GeneratedCache, "piece_slots", piece)
    wl = W.custom(seed=41, q_lens=[1, 5, 1, 3], kv_lens=[37, 64, 9, 130], page_size=16,
                  num_qo_heads=8, num_kv_heads=2, head_dim=64, q_dtype=qd, kv_dtype=kd,
                  spare_pages=4)
    if kd == "fp8":   # a scale that makes some stored values saturate at 448
        wl.kv_scale = 2.0 ** -5
    rng = np.random.default_rng(5)
    for which in ("k", "v"):
        whole = _whole_cache(wl, which)
        lazy = orun.GeneratedCache(wl, which)
        for vals, slots in _stores(wl, rng):
            A.store_kv(whole, vals, slots)
            lazy.store(vals, slots)
        every = np.arange(wl.pool_slots)
        codes = lazy.codes_at(every)
        assert codes.dtype == whole.codes.dtype
        assert np.array_equal(codes.view(np.uint8), whole.flat().view(np.uint8))
        # decoded values (what attention reads) agree bit for bit too, in any order
        order = rng.permutation(wl.pool_slots)
        assert np.array_equal(lazy.decode_slots(order), whole.decode_slots(order))
        # materialised slots serve the same codes, and slots outside still work
        lazy.materialize(order[: len(order) // 2])
        assert np.array_equal(lazy.codes_at(every).view(np.uint8), whole.flat().view(np.uint8))


@pytest.mark.parametrize("qd,kd", [("f32", "f32"), ("bf16", "bf16"), ("bf16", "fp8")])
def test_oracle_run_on_generated_cache_equals_whole_pool(qd, kd):
    """End to end: the oracle over the lazy caches after the workload's own store
    equals the oracle over whole pools stored the plain way."""
    wl = W.custom(seed=43, q_lens=[1, 6, 2], kv_lens=[50, 70, 33], page_size=16,
                  num_qo_heads=8, num_kv_heads=2, head_dim=64, q_dtype=qd, kv_dtype=kd,
                  windows=(-1, 8))
    kc, vc = _whole_cache(wl, "k"), _whole_cache(wl, "v")
    A.store_kv(kc, W.new_kv_values(wl, "k"), wl.slot_mapping)
    A.store_kv(vc, W.new_kv_values(wl, "v"), wl.slot_mapping)
    q = orun.decoded_q(wl)
    for window in wl.windows:
        o1, l1 = orun.run(wl, window=window)
        o2, l2 = A.paged_attention(q, kc, vc, wl.qo_indptr, wl.kv_indptr, wl.kv_indices,
                                   wl.last_page_len, wl.num_kv_heads, sm_scale=wl.sm_scale,
                                   causal=wl.causal, window=window)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


# ----------------------------------------------------- the value generator

def _mueller(x):
    """Thomas Mueller's 32-bit integer hash, in Python integers."""
    x &= 0xFFFFFFFF
    for _ in range(2):
        x = (((x >> 16) ^ x) * 0x45D9F3B) & 0xFFFFFFFF
    return ((x >> 16) ^ x) & 0xFFFFFFFF


def _index_py(seed, stream, c):
    """Table index of counter c, from the generator's definition: hash the low
    32 bits keyed by k1, the high bits keyed by k2, combine and hash again."""
    k1, k2 = R.stream_keys(seed, stream)
    h = _mueller((c & 0xFFFFFFFF) ^ k1)
    hi = _mueller((c >> 32) ^ k2)
    return _mueller(h ^ hi) & 0xFFFF


def test_generator_matches_its_definition():
    counters = [0, 1, 2, 12345, 2 ** 31 - 1, 2 ** 32 - 1, 2 ** 32, 2 ** 32 + 17, 3 * 2 ** 35 + 5]
    for seed, stream in ((1, "q"), (4, "k_pool"), (5005, "v_new")):
        got = R.table_index_np(seed, stream, np.asarray(counters))
        assert got.tolist() == [_index_py(seed, stream, c) for c in counters]
    # the tables: float32 normal quantiles (checked through the CDF, a different
    # routine from the quantile function that built them), bf16 = float32
    # truncated to its top 16 bits
    from scipy.special import ndtr
    u = (np.arange(65536) + 0.5) / 65536.0
    assert np.all(np.diff(R.TABLE_F32) > 0)
    assert np.max(np.abs(ndtr(R.TABLE_F32.astype(np.float64)) - u)) < 1e-7
    assert np.array_equal(R.TABLE_BF16_AS_F32.view(np.uint32) & 0xFFFF, np.zeros(65536, np.uint32))
    assert np.all(np.abs(R.TABLE_BF16_AS_F32) <= np.abs(R.TABLE_F32))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("start", [0, 1000, 2 ** 32 - 300])
def test_fill_torch_equals_values_np(dtype, start):
    n = 5000
    t = torch.empty(n, dtype=dtype)
    R.fill_torch(t, 9, "k_pool", start=start, chunk=777)     # several chunks and a ragged tail
    name = "f32" if dtype == torch.float32 else "bf16"
    ref = R.values_np(9, "k_pool", np.arange(start, start + n), name)
    assert np.array_equal(t.float().numpy(), ref)


def test_device_inputs_pool_equals_pool_values():
    wl = W.custom(seed=47, q_lens=[1, 3], kv_lens=[20, 40], page_size=16, num_qo_heads=4,
                  num_kv_heads=2, head_dim=64)
    d = W.device_inputs(wl, "cpu")
    for w in ("k", "v"):
        got = d[f"{w}_cache"].float().numpy().reshape(-1, wl.num_kv_heads, wl.head_dim)
        assert np.array_equal(got, W.pool_values(wl, w, np.arange(wl.pool_slots)))
        assert np.array_equal(d[f"{w}_new"].float().numpy(), W.new_kv_values(wl, w))
    assert np.array_equal(d["q"].float().numpy(), W.q_values(wl))
