"""store_kv on the GPU, bit-exact against the oracle's store (all five workloads,
both readings of the tiny workload's store, every dtype conversion, strided
source and cache views)."""

import numpy as np
import pytest
import torch

import paged_kv_attention_store_amd as ak
from oracle import attention as A
from oracle import codecs as C
from oracle import workload_run as orun
from synth import workloads as W
from tests.gpu_harness import prepare, say

pytestmark = pytest.mark.gpu


def _bits(t):
    t = t.cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def _cache_rows(cache, slots):
    P, B, H, D = cache.shape
    flat = cache.view(P * B, H, D)
    return _bits(flat[torch.from_numpy(np.asarray(slots)).to(cache.device)])


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
def test_store_new_tokens_bit_exact(k):
    say(f"[store] config {k}")
    wl = W.config(k)
    d = prepare(wl)
    torch.cuda.synchronize()
    kc, vc = orun.caches_after_store(wl)
    slots = wl.slot_mapping
    for w, cache, oc in (("k", d["k_cache"], kc), ("v", d["v_cache"], vc)):
        got = _cache_rows(cache, slots)
        exp = oc.codes_at(slots)
        assert np.array_equal(got.view(np.uint8), exp.view(np.uint8)), f"{w} new rows differ"
        # untouched pool rows keep their generated (and, for fp8, quantised) codes
        rng = np.random.default_rng(k)
        other = rng.choice(wl.pool_slots, size=min(2048, wl.pool_slots), replace=False)
        other = np.setdiff1d(other, slots)
        assert np.array_equal(_cache_rows(cache, other).view(np.uint8),
                              oc.codes_at(other).view(np.uint8)), f"{w} pool rows differ"


@pytest.mark.parametrize("k", [1, 2, 3])
@pytest.mark.parametrize("layout", ["fused_qkv", "head_pairs"])
def test_store_strided_views_bit_exact(k, layout):
    # Sources: K and V as slices of a fused [T, Hq + 2 Hkv, D] projection (token
    # stride wider than a row, heads contiguous), or interleaved per head
    # [T, Hkv, 2, D] (head stride 2 D).  Caches: K and V interleaved per head in
    # one pool [P, B, Hkv, 2, D] (head stride 2 D), so the kernel's general
    # (head, column) addressing runs, and the fused one on the sources.
    wl = W.config(k)
    say(f"[store] config {k}, strided views ({layout})")
    d = prepare(wl, store_new=False)
    P, B, H, D = d["k_cache"].shape
    T = d["k_new"].shape[0]
    if layout == "fused_qkv":
        Hq = wl.num_qo_heads
        fused = torch.empty(T, Hq + 2 * H, D, dtype=d["k_new"].dtype, device="cuda")
        fused[:, Hq:Hq + H] = d["k_new"]
        fused[:, Hq + H:] = d["v_new"]
        ks, vs = fused[:, Hq:Hq + H], fused[:, Hq + H:]
    else:
        pairs = torch.empty(T, H, 2, D, dtype=d["k_new"].dtype, device="cuda")
        pairs[:, :, 0] = d["k_new"]
        pairs[:, :, 1] = d["v_new"]
        ks, vs = pairs[:, :, 0], pairs[:, :, 1]
    pool = torch.empty(P, B, H, 2, D, dtype=d["k_cache"].dtype, device="cuda")
    pool[:, :, :, 0] = d["k_cache"]
    pool[:, :, :, 1] = d["v_cache"]
    kc, vc = pool[:, :, :, 0], pool[:, :, :, 1]
    assert not ks.is_contiguous() and not kc.is_contiguous()
    ak.ak_store_kv(ks, vs, d["slot_mapping"], kc, vc, wl.kv_scale, wl.kv_scale)
    torch.cuda.synchronize()
    okc, ovc = orun.caches_after_store(wl)
    slots = wl.slot_mapping
    rng = np.random.default_rng(100 + k)
    other = np.setdiff1d(rng.choice(wl.pool_slots, size=min(2048, wl.pool_slots), replace=False),
                         slots)
    for w, cache, oc in (("k", kc, okc), ("v", vc, ovc)):
        c = cache.contiguous()
        assert np.array_equal(_cache_rows(c, slots).view(np.uint8),
                              oc.codes_at(slots).view(np.uint8)), f"{w} new rows differ"
        assert np.array_equal(_cache_rows(c, other).view(np.uint8),
                              oc.codes_at(other).view(np.uint8)), f"{w} pool rows differ"


def test_tiny_store_reading_b_free_slots():
    wl = W.config(1)
    d = prepare(wl, store_new=False)
    free = wl.extra["free_slots"]
    ak.ak_store_kv(d["k_new"], d["v_new"], torch.from_numpy(free).cuda(), d["k_cache"],
                   d["v_cache"])
    torch.cuda.synchronize()
    kc, vc = orun.caches_after_store(wl, slot_mapping=free)
    # the whole pool, bit for bit
    every = np.arange(wl.pool_slots)
    assert np.array_equal(_cache_rows(d["k_cache"], every), kc.codes_at(every))
    assert np.array_equal(_cache_rows(d["v_cache"], every), vc.codes_at(every))


@pytest.mark.parametrize("src,dst", [("f32", "f32"), ("f32", "bf16"), ("f32", "fp8"),
                                     ("bf16", "bf16"), ("bf16", "fp8")])
def test_conversions_and_padding(src, dst):
    rng = np.random.default_rng(5)
    N, H, D, P, B = 300, 2, 64, 40, 16
    vals = (rng.standard_normal((N, H, D)) * rng.choice([1e-3, 1.0, 30.0, 300.0], size=(N, 1, 1)))
    vals = vals.astype(np.float32)
    # exact bf16 ties and e4m3 ties in the first rows
    vals[0, 0, :16] = ((np.arange(16, dtype=np.uint32) << 16) + 0x3F808000).view(np.float32)
    vals[1, 0, :8] = np.array([1.0625, 1.1875, 0.0048828125 * 1.5, 448.0, 464.0, -500.0,
                               2 ** -10, -(2 ** -10) * 3], dtype=np.float32)
    if src == "bf16":
        vals = C.bf16_decode(C.bf16_encode(vals)).astype(np.float32)
    scale = 0.25 if dst == "fp8" else 1.0
    slots = rng.permutation(P * B)[:N].astype(np.int64)
    slots[::7] = -1                                    # padding rows are skipped
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}
    k = torch.from_numpy(vals).to(tdt[src]).cuda() if src == "f32" else \
        torch.from_numpy(C.bf16_encode(vals).view(np.int16)).view(torch.bfloat16).cuda()
    v = -k
    kc = torch.zeros(P, B, H, D, dtype=tdt[dst], device="cuda")
    vc = torch.zeros_like(kc)
    ak.ak_store_kv(k, v, torch.from_numpy(slots).cuda(), kc, vc, scale, scale)
    torch.cuda.synchronize()
    zero = np.zeros((P, B, H, D), dtype=np.float32)
    for sign, cache in ((1, kc), (-1, vc)):
        oc = A.Cache(A.encode(zero, dst, scale), dst, scale)
        A.store_kv(oc, sign * vals, slots)
        got = _bits(cache).reshape(-1)
        assert np.array_equal(got.view(np.uint8), oc.codes.reshape(-1).view(np.uint8))


def test_store_rejects_bad_arguments():
    k = torch.zeros(4, 2, 64, dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros(2, 16, 2, 64, dtype=torch.bfloat16, device="cuda")
    s32 = torch.zeros(4, dtype=torch.int32, device="cuda")
    with pytest.raises(ak.AkError) as e:
        ak.ak_store_kv(k, k, s32, kc, kc.clone())
    assert e.value.status == ak.AK_ERR_UNSUPPORTED
    kf = torch.zeros(2, 16, 2, 64, dtype=torch.float32, device="cuda")
    s64 = torch.zeros(4, dtype=torch.int64, device="cuda")
    with pytest.raises(ak.AkError) as e:           # bf16 -> f32 widening is not a store
        ak.ak_store_kv(k, k, s64, kf, kf.clone())
    assert e.value.status == ak.AK_ERR_UNSUPPORTED
    with pytest.raises(ak.AkError) as e:
        ak.ak_store_kv(k, k, s64[:3], kc, kc.clone())
    assert e.value.status == ak.AK_ERR_SHAPE_MISMATCH


def test_fp8_widening_exhaustive():
    """The kernels' E4M3 -> bf16 widening on every finite code equals the format
    definition (oracle decode table), bit for bit."""
    codes = np.arange(256, dtype=np.uint8)
    finite = np.isfinite(C.E4M3_VALUES)
    codes = np.tile(codes[finite], 4)            # 254 finite codes, length a multiple of 8
    codes = codes[: len(codes) // 8 * 8]
    got = ak.ak_fp8_to_bf16(torch.from_numpy(codes).cuda())
    torch.cuda.synchronize()
    got_bits = got.cpu().view(torch.int16).numpy().view(np.uint16)
    exp_bits = C.bf16_encode(C.e4m3_decode(codes).astype(np.float32))
    assert np.array_equal(got_bits, exp_bits)


def _draw_store(seed: int):
    """A seeded store: token count (0 to 5000, one empty store, one case past the
    launch's 8192-block cap so the grid-stride loop runs), heads, head size, page size,
    dtype pair, per-tensor scale, value magnitudes from 2^-20 to 600 (fp8
    saturation and subnormals included) and 0-20% padding slots."""
    rng = np.random.default_rng(4200 + seed)
    N = 40000 if seed == 0 else int(rng.integers(0, 5001))
    if seed == 11:
        N = 0
    H = int(rng.choice([1, 3, 8]))
    D = int(rng.choice([8, 64, 128, 256]))
    if seed == 0:
        H, D = 1, 64
    B = int(rng.choice([1, 16, 64]))
    P = (N + B - 1) // B + int(rng.integers(1, 9))
    src, dst = [("f32", "f32"), ("f32", "bf16"), ("f32", "fp8"), ("bf16", "bf16"),
                ("bf16", "fp8")][int(rng.integers(5))]
    scale = float(2.0 ** rng.uniform(-5, 2)) if dst == "fp8" else 1.0
    mag = 2.0 ** rng.uniform(-20, np.log2(600), size=(N, H, 1))
    vals = (rng.standard_normal((N, H, D)) * mag).astype(np.float32)
    slots = rng.permutation(P * B)[:N].astype(np.int64)
    slots[rng.random(N) < rng.uniform(0, 0.2)] = -1
    return N, H, D, P, B, src, dst, scale, vals, slots


@pytest.mark.parametrize("seed", range(12))
def test_store_random_shapes_bit_exact(seed):
    N, H, D, P, B, src, dst, scale, vals, slots = _draw_store(seed)
    say(f"[store] random {seed}: N={N} H={H} D={D} P={P} B={B} {src}->{dst} scale={scale:.4g}")
    if src == "bf16":
        vals = C.bf16_decode(C.bf16_encode(vals)).astype(np.float32)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}
    if src == "f32":
        k = torch.from_numpy(vals).cuda()
    else:
        k = torch.from_numpy(C.bf16_encode(vals).view(np.int16)).view(torch.bfloat16).cuda()
    v = -k
    kc = torch.zeros(P, B, H, D, dtype=tdt[dst], device="cuda")
    vc = torch.zeros_like(kc)
    ak.ak_store_kv(k, v, torch.from_numpy(slots).cuda(), kc, vc, scale, scale)
    torch.cuda.synchronize()
    zero = np.zeros((P, B, H, D), dtype=np.float32)
    for sign, cache in ((1, kc), (-1, vc)):
        oc = A.Cache(A.encode(zero, dst, scale), dst, scale)
        A.store_kv(oc, sign * vals, slots)
        got = _bits(cache).reshape(-1)
        assert np.array_equal(got.view(np.uint8), oc.codes.reshape(-1).view(np.uint8))
