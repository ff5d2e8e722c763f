"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each test names what it pins against: a page's printed worked example (JSON
fixtures under tests/golden/, each with its source), a library routine on a
special case, brute force on tiny inputs, or a closed form.  The planted-mistake
tests at the end change one oracle step to a plausible wrong version and check
that some pin fails.
"""

import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import attention as A
from oracle import codecs as C
from oracle import metadata as M

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ------------------------------------------------ worked example, vLLM page

def test_vllm_worked_example_csr_and_slots():
    g = _gold("vllm_worked_example.json")
    e = g["expect"]
    B = g["page_size"]
    qsl = np.asarray(g["query_start_loc"])
    seq = g["seq_lens"]
    rows = g["block_rows"]
    indptr, indices, last = M.block_table_to_csr(seq, rows, B)
    assert indptr.tolist() == e["paged_kv_indptr"]
    assert indices.tolist() == e["paged_kv_indices"]
    assert last.tolist() == e["paged_kv_last_page_len"]
    assert (indptr[1:] - indptr[:-1]).tolist() == e["pages_per_request"]
    qlen = M.q_lengths(qsl)
    positions = [range(s - n, s) for s, n in zip(seq, qlen)]
    assert M.slot_mapping(rows, positions, B).tolist() == e["slot_mapping"]
    dec, dec_ptr, pre, pre_ptr = M.split_decode_prefill(qsl, threshold=1)
    assert len(dec) == e["num_decodes"] and int(dec_ptr[-1]) == e["num_decode_tokens"]
    assert len(pre) == e["num_prefills"] and int(pre_ptr[-1]) == e["num_prefill_tokens"]
    assert pre_ptr.tolist() == e["prefill_qo_indptr"]
    # the reverse direction: lengths recovered from the CSR arrays
    assert M.kv_lengths(indptr, last, B).tolist() == seq


def test_vllm_worked_example_slices_cover_every_token_once():
    g = _gold("vllm_worked_example.json")
    qsl = np.asarray(g["query_start_loc"])
    dec, dec_ptr, pre, pre_ptr = M.split_decode_prefill(qsl)
    covered = []
    for ids in (dec, pre):
        for r in ids:
            covered.extend(range(int(qsl[r]), int(qsl[r + 1])))
    assert sorted(covered) == list(range(int(qsl[-1])))


def test_virtual_blocks_of_the_pages_example():
    # a 64-token manager block seen as four 16-token kernel blocks: manager
    # blocks 5 and 2 are kernel pages 20..23 and 8..11 of the 16-token view
    assert M.virtual_block_rows([[5, 2]], 4) == [[20, 21, 22, 23, 8, 9, 10, 11]]
    assert M.virtual_block_rows([[7, 0, 3]], 1) == [[7, 0, 3]]


@pytest.mark.parametrize("ratio", [1, 2, 4, 8])
def test_virtual_blocks_keep_every_flat_slot(ratio):
    # the expansion is a relabelling of one memory: position p of a request has
    # the same flat slot through M-token manager blocks and B-token kernel pages
    # (slot_of is pinned by the vLLM worked example)
    rng = np.random.default_rng(ratio)
    B = 16
    Mtok = ratio * B
    rows = [rng.permutation(50)[:k].tolist() for k in (1, 3, 7)]
    vrows = M.virtual_block_rows(rows, ratio)
    for row, vrow in zip(rows, vrows):
        L = len(row) * Mtok
        for p in range(L):
            assert M.slot_of(row, p, Mtok) == M.slot_of(vrow, p, B)
    # and the CSR built from kernel pages gathers the same slots as the one built
    # from manager blocks
    lens = [5, 3 * Mtok - 1, 7 * Mtok]
    i1, x1, l1 = M.block_table_to_csr(lens, rows, Mtok)
    i2, x2, l2 = M.block_table_to_csr(lens, vrows, B)
    for r in range(3):
        assert np.array_equal(M.request_slots(i1, x1, l1, Mtok, r),
                              M.request_slots(i2, x2, l2, B, r))


def test_last_page_len_never_zero():
    # a full last page is B, not 0 (CSR section of the vLLM page)
    for B in (1, 2, 16, 64):
        for l in range(1, 4 * B + 1):
            _, _, last = M.block_table_to_csr([l], [list(range(8))], B)
            assert 1 <= last[0] <= B
            assert (math.ceil(l / B) - 1) * B + last[0] == l


# --------------------------------------------- worked example, mini-sglang

def _minisglang_metadata():
    g = _gold("minisglang_example.json")
    rows = g["token_table_rows"]
    L = g["prompt_lens"]
    cached = g["cached_lens"]
    n = [l - c for l, c in zip(L, cached)]
    qo = np.concatenate([[0], np.cumsum(n)])
    return g, rows, L, n, qo


def test_minisglang_page_size_1_view():
    g, rows, L, n, qo = _minisglang_metadata()
    e = g["expect"]["page_size_1"]
    indptr, indices, last = M.block_table_to_csr(L, rows, 1)
    assert qo.tolist() == e["qo_indptr"]
    assert indptr.tolist() == e["kv_indptr"]
    assert indices.tolist() == e["kv_indices"]
    assert last.tolist() == e["last_page_len"]


def test_minisglang_page_size_4_view():
    g, rows, L, n, qo = _minisglang_metadata()
    e = g["expect"]["page_size_4"]
    assert M.page_table_from_token_table(rows, L, 4) == e["page_table"]
    assert qo.tolist() == e["cu_seqlens_q"]
    indptr, indices, last = M.block_table_to_csr(L, e["page_table"], 4)
    assert M.kv_lengths(indptr, last, 4).tolist() == e["cache_seqlens"]


def _pool(rng, tokens, hkv, d):
    return rng.standard_normal((tokens, hkv, d)).astype(np.float32)


def test_minisglang_page_view_equals_token_view_bitwise():
    """Same pool read through B=4 page numbers and through B=1 token slots gives
    bit-identical out and lse (the page prints 0.00e+00 for both backends)."""
    g, rows, L, n, qo = _minisglang_metadata()
    rng = np.random.default_rng(7)
    hq, hkv, d = 4, 2, 8
    kp, vp = _pool(rng, g["pool_tokens"], hkv, d), _pool(rng, g["pool_tokens"], hkv, d)
    q = rng.standard_normal((int(qo[-1]), hq, d))
    # token view
    i1, x1, l1 = M.block_table_to_csr(L, rows, 1)
    kc1 = A.Cache(kp.reshape(-1, 1, hkv, d), "f32")
    vc1 = A.Cache(vp.reshape(-1, 1, hkv, d), "f32")
    o1, s1 = A.paged_attention(q, kc1, vc1, qo, i1, x1, l1, hkv)
    # page view of the same memory
    pt = M.page_table_from_token_table(rows, L, 4)
    i4, x4, l4 = M.block_table_to_csr(L, pt, 4)
    kc4 = A.Cache(kp.reshape(-1, 4, hkv, d), "f32")
    vc4 = A.Cache(vp.reshape(-1, 4, hkv, d), "f32")
    o4, s4 = A.paged_attention(q, kc4, vc4, qo, i4, x4, l4, hkv)
    assert np.array_equal(o1, o4) and np.array_equal(s1, s4)
    assert float(np.max(np.abs(o1 - o4))) == g["expect"]["max_abs_diff_between_views"]
    # and the page view -> token view rewrite reproduces the B=1 CSR
    ti, tx, tl = M.token_view(i4, x4, l4, 4)
    assert ti.tolist() == i1.tolist() and tx.tolist() == x1.tolist() and tl.tolist() == [1, 1]


# ------------------------------------------- library routine: torch SDPA

def _contiguous_case(rng, L, n, hq, hkv, d):
    """One request whose pages are 0, 1, 2, ... (identity page table)."""
    B = 4
    pages = -(-L // B)
    kpool = rng.standard_normal((pages * B, hkv, d))
    vpool = rng.standard_normal((pages * B, hkv, d))
    q = rng.standard_normal((n, hq, d))
    indptr = np.array([0, pages])
    indices = np.arange(pages)
    last = np.array([L - (pages - 1) * B])
    qo = np.array([0, n])
    kc = A.Cache(kpool.reshape(pages, B, hkv, d), "f32")
    vc = A.Cache(vpool.reshape(pages, B, hkv, d), "f32")
    kc.decode_slots = lambda s, p=kpool: p[np.asarray(s)]   # keep float64 inputs exact
    vc.decode_slots = lambda s, p=vpool: p[np.asarray(s)]
    return q, kc, vc, qo, indptr, indices, last, kpool[:L], vpool[:L]


@pytest.mark.parametrize("L,n,hq,hkv,causal,window", [
    (9, 1, 4, 2, True, -1), (9, 9, 4, 2, True, -1), (13, 5, 8, 2, True, -1),
    (13, 5, 4, 4, True, -1), (13, 5, 8, 1, False, -1), (17, 6, 4, 2, True, 3),
    (17, 6, 8, 4, True, 0), (6, 6, 2, 2, True, 2),
])
def test_against_torch_sdpa_fp64(L, n, hq, hkv, causal, window):
    rng = np.random.default_rng(L * 100 + n)
    d = 16
    q, kc, vc, qo, indptr, indices, last, K, V = _contiguous_case(rng, L, n, hq, hkv, d)
    scale = 1 / math.sqrt(d)
    out, lse = A.paged_attention(q, kc, vc, qo, indptr, indices, last, hkv, sm_scale=scale,
                                 causal=causal, window=window)
    # explicit bottom-right boolean mask handed to the library routine
    qpos = torch.arange(L - n, L).unsqueeze(1)
    t = torch.arange(L).unsqueeze(0)
    mask = torch.ones(n, L, dtype=torch.bool)
    if causal:
        mask &= t <= qpos
    if window >= 0:
        mask &= t >= qpos - window
    ref = F.scaled_dot_product_attention(
        torch.from_numpy(q).transpose(0, 1), torch.from_numpy(K).transpose(0, 1).contiguous(),
        torch.from_numpy(V).transpose(0, 1).contiguous(), attn_mask=mask, scale=scale,
        enable_gqa=(hq != hkv)).transpose(0, 1).numpy()
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


# -------------------------------------------------- brute force, tiny sizes

def _brute(q, K, V, scale, causal, window):
    """Dense softmax attention with Python floats, rows = queries at the end."""
    n, L = len(q), len(K)
    outs, lses = [], []
    for j in range(n):
        pos = L - n + j
        vis = [t for t in range(L) if (not causal or t <= pos) and (window < 0 or t >= pos - window)]
        s = {t: scale * sum(a * b for a, b in zip(q[j], K[t])) for t in vis}
        m = max(s.values())
        w = {t: math.exp(s[t] - m) for t in vis}
        z = sum(w.values())
        outs.append([sum(w[t] * V[t][c] for t in vis) / z for c in range(len(V[0]))])
        lses.append(m + math.log(z))
    return outs, lses


@pytest.mark.parametrize("L,n,causal,window", [(8, 8, True, -1), (8, 3, True, 2), (5, 1, False, -1),
                                               (7, 4, False, -1), (8, 8, True, 0)])
def test_brute_force_tiny(L, n, causal, window):
    rng = np.random.default_rng(11 + L + n)
    d = 4
    q, kc, vc, qo, indptr, indices, last, K, V = _contiguous_case(rng, L, n, 2, 1, d)
    scale = 0.7
    out, lse = A.paged_attention(q, kc, vc, qo, indptr, indices, last, 1, sm_scale=scale,
                                 causal=causal, window=window)
    for h in range(2):
        bo, bl = _brute(q[:, h, :].tolist(), K[:, 0, :].tolist(), V[:, 0, :].tolist(), scale,
                        causal, window)
        np.testing.assert_allclose(out[:, h, :], np.array(bo), rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[:, h], np.array(bl), rtol=0, atol=1e-13)


# ------------------------------------------------------------ closed forms

def test_constant_values_give_constant_output():
    rng = np.random.default_rng(3)
    q, kc, vc, qo, indptr, indices, last, K, V = _contiguous_case(rng, 23, 5, 4, 2, 8)
    const = np.full((32, 2, 8), 0.375)
    vc.decode_slots = lambda s: const[np.asarray(s)]
    out, _ = A.paged_attention(q, kc, vc, qo, indptr, indices, last, 2, causal=True, window=4)
    assert np.all(np.abs(out - 0.375) < 1e-15)


def test_equal_keys_give_uniform_weights():
    rng = np.random.default_rng(4)
    L, n, d = 12, 4, 8
    q, kc, vc, qo, indptr, indices, last, K, V = _contiguous_case(rng, L, n, 2, 1, d)
    key = rng.standard_normal(d)
    Kc = np.tile(key, (len(K) + 4, 1, 1)).reshape(-1, 1, d)
    kc.decode_slots = lambda s: Kc[np.asarray(s)]
    scale = 0.3
    for window in (-1, 2):
        out, lse = A.paged_attention(q, kc, vc, qo, indptr, indices, last, 1, sm_scale=scale,
                                     causal=True, window=window)
        for j in range(n):
            pos = L - n + j
            lo = 0 if window < 0 else max(0, pos - window)
            cnt = pos - lo + 1
            for h in range(2):
                s0 = scale * float(q[j, h] @ key)
                np.testing.assert_allclose(lse[j, h], s0 + math.log(cnt), atol=1e-12)
                np.testing.assert_allclose(out[j, h], V[lo:pos + 1, 0].mean(axis=0), atol=1e-12)


def test_wide_window_equals_no_window_and_decode_ignores_causal():
    rng = np.random.default_rng(5)
    L = 19
    q, kc, vc, qo, indptr, indices, last, K, V = _contiguous_case(rng, L, 6, 4, 2, 8)
    a = A.paged_attention(q, kc, vc, qo, indptr, indices, last, 2, causal=True, window=-1)
    b = A.paged_attention(q, kc, vc, qo, indptr, indices, last, 2, causal=True, window=L)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    q1 = q[-1:]
    c = A.paged_attention(q1, kc, vc, np.array([0, 1]), indptr, indices, last, 2, causal=True)
    d = A.paged_attention(q1, kc, vc, np.array([0, 1]), indptr, indices, last, 2, causal=False)
    assert np.array_equal(c[0], d[0]) and np.array_equal(c[1], d[1])


# ----------------------------------------------------------- split + merge

@pytest.mark.parametrize("cuts", [[0, 7, 30], [0, 1, 2, 30], [0, 15, 16, 17, 30], [0, 29, 30]])
def test_merge_of_any_partition_equals_unsplit(cuts):
    rng = np.random.default_rng(len(cuts))
    L, n = 30, 3
    q, kc, vc, qo, indptr, indices, last, K, V = _contiguous_case(rng, L, n, 4, 2, 8)
    full_o, full_l = A.paged_attention(q, kc, vc, qo, indptr, indices, last, 2, causal=True,
                                       window=20)
    parts = [A.paged_attention(q, kc, vc, qo, indptr, indices, last, 2, causal=True, window=20,
                               kv_range_of=lambda r, a=a, b=b: (a, b))
             for a, b in zip(cuts[:-1], cuts[1:])]
    mo, ml = A.merge_states([p[0] for p in parts], [p[1] for p in parts])
    np.testing.assert_allclose(mo, full_o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(ml, full_l, rtol=0, atol=1e-12)


def test_merge_is_associative_and_ignores_empty_parts():
    rng = np.random.default_rng(9)
    o = [rng.standard_normal((5, 8)) for _ in range(3)]
    s = [rng.standard_normal(5) * 3 for _ in range(3)]
    ab = A.merge_states(o[:2], s[:2])
    left = A.merge_states([ab[0], o[2]], [ab[1], s[2]])
    bc = A.merge_states(o[1:], s[1:])
    right = A.merge_states([o[0], bc[0]], [s[0], bc[1]])
    np.testing.assert_allclose(left[0], right[0], atol=1e-13)
    np.testing.assert_allclose(left[1], right[1], atol=1e-13)
    e = A.merge_states([o[0], np.zeros((5, 8))], [s[0], np.full(5, -np.inf)])
    np.testing.assert_allclose(e[0], o[0], atol=1e-15)
    np.testing.assert_allclose(e[1], s[0], atol=1e-15)


# ------------------------------------------------------------------ codecs

def test_bf16_encode_matches_torch_cast():
    rng = np.random.default_rng(12)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(20000) * 1e-38).astype(np.float32),     # subnormals
        (rng.standard_normal(20000) * 1e30).astype(np.float32),
        # exact ties: bf16 value + half an ulp of bf16 (low 16 bits = 0x8000)
        ((rng.integers(0, 2 ** 16, 20000).astype(np.uint32) << 16) | 0x8000).view(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38], dtype=np.float32)])
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(C.bf16_encode(x), ref)
    assert np.array_equal(C.bf16_decode(ref), torch.from_numpy(ref.view(np.int16)).view(
        torch.bfloat16).to(torch.float64).numpy())


def _all_bf16_within(limit):
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = C.bf16_decode(b)
    keep = np.isfinite(v) & (np.abs(v) <= limit)
    return b[keep], v[keep].astype(np.float32)


def test_e4m3_encode_exhaustive_over_bf16_matches_torch():
    _, v = _all_bf16_within(448.0)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(C.e4m3_encode_unit(v), ref)


def test_e4m3_encode_with_scale_matches_torch():
    rng = np.random.default_rng(13)
    x = rng.standard_normal(300000).astype(np.float32)
    scale = np.float32(np.max(np.abs(x)) / np.float32(448.0))
    ref = torch.from_numpy(x / scale).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(C.e4m3_encode(x, scale), ref)


def test_e4m3_decode_table():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = C.e4m3_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours)) and nan.sum() == 2     # 0x7F, 0xFF
    assert np.array_equal(ours[~nan], ref[~nan])
    assert C.E4M3_VALUES[0x7E] == 448.0 and C.E4M3_VALUES[0x08] == 2.0 ** -6
    assert C.E4M3_VALUES[0x01] == 2.0 ** -9
    pos = C.E4M3_VALUES[:0x7F]
    assert np.all(np.diff(pos) > 0)


def test_e4m3_saturates_and_keeps_sign():
    x = np.array([449.0, 464.0, 480.0, 1e6, -500.0, -1e-12, 0.0, -0.0], dtype=np.float32)
    got = C.e4m3_encode_unit(x)
    assert got.tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x80, 0x00, 0x80]


def test_bf16_values_decode_exactly_from_e4m3():
    # every finite E4M3 value is a bf16 value: 3 mantissa bits, exponents 2^-9 .. 2^8
    v = C.E4M3_VALUES[np.isfinite(C.E4M3_VALUES)]
    assert np.array_equal(C.bf16_decode(C.bf16_encode(v.astype(np.float32))), v)


# ------------------------------------------------ store then attend (small)

def test_store_kv_writes_in_order_and_skips_padding():
    cache = A.Cache(np.zeros((2, 4, 1, 2), dtype=np.float32), "f32")
    vals = np.arange(10, dtype=np.float32).reshape(5, 1, 2)
    A.store_kv(cache, vals, np.array([3, -1, 7, 0, 3]))
    flat = cache.flat()
    assert flat[3].tolist() == [[8.0, 9.0]]        # the later write to slot 3 wins
    assert flat[7].tolist() == [[4.0, 5.0]] and flat[0].tolist() == [[6.0, 7.0]]
    assert np.count_nonzero(flat) == 6             # token 0's write to slot 3 was overwritten
    assert np.all(flat[[1, 2, 4, 5, 6]] == 0)


# ------------------------------------------------- generator vs oracle CSR

@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
def test_workload_csr_agrees_with_oracle_metadata(k):
    from synth import workloads as W

    wl = W.config(k)
    assert M.kv_lengths(wl.kv_indptr, wl.last_page_len, wl.page_size).tolist() == wl.kv_lens.tolist()
    assert M.q_lengths(wl.qo_indptr).tolist() == wl.q_lens.tolist()
    indptr, indices, last = M.block_table_to_csr(wl.kv_lens, wl.req_pages, wl.page_size)
    assert indptr.tolist() == wl.kv_indptr.tolist() and indices.tolist() == wl.kv_indices.tolist()
    assert last.tolist() == wl.last_page_len.tolist()
    positions = [range(int(L) - int(n), int(L)) for L, n in zip(wl.kv_lens, wl.q_lens)]
    assert M.slot_mapping(wl.req_pages, positions, wl.page_size).tolist() == wl.slot_mapping.tolist()
    assert len(set(wl.kv_indices.tolist())) == len(wl.kv_indices)     # pages owned once


# ------------------------------------------------------- planted mistakes

def test_planted_kv_length_mistake_is_caught(monkeypatch):
    g = _gold("vllm_worked_example.json")
    wrong = lambda indptr, last, B: (np.diff(np.asarray(indptr)) * B + np.asarray(last))  # noqa
    monkeypatch.setattr(M, "kv_lengths", wrong)
    indptr, _, last = M.block_table_to_csr(g["seq_lens"], g["block_rows"], g["page_size"])
    assert M.kv_lengths(indptr, last, g["page_size"]).tolist() != g["seq_lens"]


def test_planted_gqa_map_mistake_is_caught():
    rng = np.random.default_rng(21)
    L, n, hq, hkv, d = 13, 5, 8, 2, 16
    q, kc, vc, qo, indptr, indices, last, K, V = _contiguous_case(rng, L, n, hq, hkv, d)
    out, _ = A.paged_attention(q, kc, vc, qo, indptr, indices, last, hkv, causal=True)
    # a modulo head map equals the right map applied to permuted query heads
    perm = np.array([(h % hkv) * (hq // hkv) + h // hkv for h in range(hq)])
    inv = np.argsort(perm)
    bad, _ = A.paged_attention(q[:, inv, :], kc, vc, qo, indptr, indices, last, hkv, causal=True)
    assert not np.allclose(bad[:, perm, :], out, atol=1e-6)


def test_planted_top_left_causal_mistake_is_caught():
    rng = np.random.default_rng(22)
    L, n = 11, 4
    q, kc, vc, qo, indptr, indices, last, K, V = _contiguous_case(rng, L, n, 2, 1, 8)
    out, _ = A.paged_attention(q, kc, vc, qo, indptr, indices, last, 1, causal=True)
    bo, _ = _brute(q[:, 0].tolist(), K[:, 0].tolist(), V[:, 0].tolist(), 1 / math.sqrt(8), True, -1)
    assert np.allclose(out[:, 0], bo, atol=1e-12)
    # top-left alignment (query j at position j) would see fewer keys
    tl = [_brute([q[j, 0].tolist()], K[:j + 1, 0].tolist(), V[:j + 1, 0].tolist(),
                 1 / math.sqrt(8), True, -1)[0][0] for j in range(n)]
    assert not np.allclose(out[:, 0], np.array(tl), atol=1e-6)


def test_planted_tie_rule_mistake_is_caught():
    _, v = _all_bf16_within(448.0)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # rounding half away from zero instead of half to even
    y = v.astype(np.float64)
    a = np.abs(y)
    grid = C.E4M3_VALUES[:0x7F]
    hi = np.clip(np.searchsorted(grid, a), 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    away = np.where((grid[hi] - a) <= (a - grid[lo]), hi, lo) | (np.signbit(y) << 7)
    assert not np.array_equal(away.astype(np.uint8), ref)
