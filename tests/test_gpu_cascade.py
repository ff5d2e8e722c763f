"""Merging attention states, and the two compositions it serves (GPU vs oracle):

* ak_merge_states against the oracle's merge ("SGLang attention backend", "The
  two forms of extend"), including states without any visible key and an
  in-place merge;
* two-segment extend: the new tokens attend to the cached prefix (paged,
  causal = 0) and to themselves (a ragged page-size-1 view of the step's new
  K/V, causal = 1); the merge equals one-pass extend attention;
* shared-prefix cascade: decode requests whose page lists start with the same
  pages attend to the shared prefix once (one non-causal request holding every
  query) and to their own suffix; the merge equals plain decode attention.
"""

import numpy as np
import pytest
import torch

import paged_kv_attention_store_amd as ak
from oracle import attention as A
from synth import workloads as W

from gpu_harness import TOL, check, prepare, say

pytestmark = pytest.mark.gpu


def _states(T, H, D, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    oa = torch.randn(T, H, D, generator=g).to(dtype)
    ob = torch.randn(T, H, D, generator=g).to(dtype)
    la = (torch.randn(T, H, generator=g) * 3).float()
    lb = (torch.randn(T, H, generator=g) * 3).float()
    # rows without a visible key in one part, in the other, and in both
    la[0, :] = -float("inf")
    lb[1, :] = -float("inf")
    la[2, 0] = lb[2, 0] = -float("inf")
    return oa, la, ob, lb


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_merge_states_matches_oracle(D, dtype):
    T, H = 37, 8
    oa, la, ob, lb = _states(T, H, D, dtype, seed=D + (dtype == torch.float32))
    ro, rl = A.merge_states([oa.double().numpy(), ob.double().numpy()],
                            [la.double().numpy(), lb.double().numpy()])
    dev = [x.cuda() for x in (oa, la, ob, lb)]
    out, lse = ak.ak_merge_states(*dev)
    torch.cuda.synchronize()
    go = out.float().cpu().double().numpy()
    gl = lse.cpu().double().numpy()
    # fp32: a few ulps of fp32 arithmetic; bf16: the output's own rounding (half a
    # bf16 ulp, 2^-9 relative) plus fp32 arithmetic -- bounded by one bf16 ulp
    rel = 1e-6 if dtype == torch.float32 else 2.0 ** -8
    assert np.all(np.abs(go - ro) <= rel * np.maximum(np.abs(ro), 1.0))
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(gl), fin) and np.max(np.abs(gl[fin] - rl[fin])) <= 1e-4
    assert np.all(go[2, 0] == 0.0)                       # both parts empty: zero row
    # in place: out is o_a and lse_out is lse_a
    ak.ak_merge_states(dev[0], dev[1], dev[2], dev[3], out=dev[0], lse_out=dev[1])
    torch.cuda.synchronize()
    assert torch.equal(dev[0].cpu(), out.cpu())
    assert torch.equal(dev[1].cpu(), lse.cpu())


def test_merge_states_rejects_bad_arguments():
    oa, la, ob, lb = [x.cuda() for x in _states(4, 2, 128, torch.bfloat16, seed=3)]
    with pytest.raises(ak.AkError) as e:
        ak.ak_merge_states(oa, la, ob[:3], lb)
    assert e.value.status == ak.AK_ERR_SHAPE_MISMATCH
    with pytest.raises(ak.AkError) as e:
        ak.ak_merge_states(oa, la, ob.float(), lb)
    assert e.value.status == ak.AK_ERR_UNSUPPORTED
    with pytest.raises(ak.AkError) as e:
        ak.ak_merge_states(oa[..., :96].contiguous(), la, ob[..., :96].contiguous(), lb)
    assert e.value.status == ak.AK_ERR_UNSUPPORTED


def _prefix_csr(wl):
    """CSR of each request's cached prefix (positions 0 .. L_r - n_r - 1)."""
    B = wl.page_size
    kv_indptr, idx, last = [0], [], []
    for r in range(wl.batch_size):
        p = int(wl.kv_lens[r] - wl.q_lens[r])
        pages = -(-p // B)
        idx.extend(wl.kv_indices[wl.kv_indptr[r]:wl.kv_indptr[r] + pages].tolist())
        kv_indptr.append(kv_indptr[-1] + pages)
        last.append(p - (pages - 1) * B if pages else 0)
    return (np.asarray(kv_indptr, np.int32), np.asarray(idx, np.int32),
            np.asarray(last, np.int32))


@pytest.mark.parametrize("case", [
    # q_lens, kv_lens (prefix = L - n), page size, heads, D
    ([17, 300, 1, 64], [100, 310, 40, 64 + 700], 16, 32, 8, 128),
    ([5, 130, 2], [6, 1130, 70], 1, 16, 4, 64),
    ([260, 3], [260, 3], 16, 8, 2, 128),       # no cached prefix: the prefix state is empty
], ids=["mixed", "page1_d64", "no_prefix"])
def test_two_segment_extend_equals_one_pass(case):
    ql, kl, B, hq, hkv, D = case
    wl = W.custom(seed=sum(kl) + B, q_lens=ql, kv_lens=kl, page_size=B, num_qo_heads=hq,
                  num_kv_heads=hkv, head_dim=D, name="two_segment")
    say(f"[two-segment] {ql} over {kl}, B={B}")
    d = prepare(wl)
    T = wl.total_q
    # segment 1: the cached prefix, every key visible to every new token
    pi, px, pl = _prefix_csr(wl)
    p1 = ak.ak_plan(wl.qo_indptr, pi, torch.from_numpy(px).cuda(), pl, hq, hkv, D, B,
                    causal=False)
    o1, l1 = ak.ak_run(p1, d["q"], d["k_cache"], d["v_cache"],
                       lse=torch.empty(T, hq, device="cuda"))
    # segment 2: the step's new K/V as a ragged page-size-1 cache, causal among themselves
    kn = d["k_new"].view(T, 1, hkv, D)
    vn = d["v_new"].view(T, 1, hkv, D)
    p2 = ak.ak_plan(wl.qo_indptr, wl.qo_indptr, torch.arange(T, dtype=torch.int32, device="cuda"),
                    np.ones(wl.batch_size, np.int32), hq, hkv, D, 1, causal=True)
    o2, l2 = ak.ak_run(p2, d["q"], kn, vn, lse=torch.empty(T, hq, device="cuda"))
    out, lse = ak.ak_merge_states(o1, l1, o2, l2)
    torch.cuda.synchronize()
    check(wl, out, lse, -1)


@pytest.mark.parametrize("case", [
    # requests, KV lengths range, shared pages, page size, heads
    (24, (300, 900), 12, 16, 32, 8),
    (40, (2100, 4000), 128, 16, 32, 8),      # long shared prefix: split across CUs
    (8, (70, 200), 1, 64, 16, 2),
], ids=["short", "long_prefix", "one_page"])
def test_shared_prefix_cascade_equals_decode(case):
    R, (lo, hi), k, B, hq, hkv = case
    D = 128
    rng = np.random.default_rng(R * 7 + k)
    kl = rng.integers(max(lo, k * B + 2), hi, size=R)
    wl = W.custom(seed=R + k, q_lens=np.ones(R, np.int64), kv_lens=kl, page_size=B,
                  num_qo_heads=hq, num_kv_heads=hkv, head_dim=D, name="cascade")
    # every request's page list starts with request 0's first k pages
    for r in range(1, R):
        wl.kv_indices[wl.kv_indptr[r]:wl.kv_indptr[r] + k] = wl.kv_indices[:k]
    say(f"[cascade] R={R} L={kl.min()}..{kl.max()} shared {k} pages of {B}")
    d = prepare(wl)
    T = wl.total_q
    # the shared prefix once: one request holding every query, no causal mask
    ps = ak.ak_plan([0, T], [0, k], torch.from_numpy(wl.kv_indices[:k].copy()).cuda(), [B],
                    hq, hkv, D, B, causal=False)
    o1, l1 = ak.ak_run(ps, d["q"], d["k_cache"], d["v_cache"],
                       lse=torch.empty(T, hq, device="cuda"))
    # each request's own suffix pages
    sx = np.concatenate([wl.kv_indices[wl.kv_indptr[r] + k:wl.kv_indptr[r + 1]] for r in range(R)])
    si = np.concatenate([[0], np.cumsum(np.diff(wl.kv_indptr) - k)]).astype(np.int32)
    p2 = ak.ak_plan(wl.qo_indptr, si, torch.from_numpy(sx.astype(np.int32)).cuda(),
                    wl.last_page_len, hq, hkv, D, B, causal=True)
    o2, l2 = ak.ak_run(p2, d["q"], d["k_cache"], d["v_cache"],
                       lse=torch.empty(T, hq, device="cuda"))
    out, lse = ak.ak_merge_states(o1, l1, o2, l2)
    torch.cuda.synchronize()
    check(wl, out, lse, -1)
    # plain decode of the same batch with cached (shared-pages) and streamed K/V
    # reads: the flag changes cache behaviour only, so the bits are the same
    runs = []
    for shared in (True, False):
        pl = ak.ak_plan(wl.qo_indptr, wl.kv_indptr, d["kv_indices"], wl.last_page_len, hq, hkv, D,
                        B, shared_pages=shared)
        runs.append(ak.ak_run(pl, d["q"], d["k_cache"], d["v_cache"],
                              lse=torch.empty(T, hq, device="cuda")))
    torch.cuda.synchronize()
    assert torch.equal(runs[0][0], runs[1][0]) and torch.equal(runs[0][1], runs[1][1])
    check(wl, runs[0][0], runs[0][1], -1)


def test_noncausal_more_queries_than_keys():
    # non-causal requests with n > L and one without pages (its rows: out 0, lse -inf)
    wl = W.custom(seed=77, q_lens=[40, 3, 300], kv_lens=[25, 0, 90], page_size=16,
                  num_qo_heads=8, num_kv_heads=2, head_dim=128, causal=False, name="nc_short")
    say("[noncausal] n > L and L = 0")
    d = prepare(wl)
    T = wl.total_q
    plan = ak.ak_plan(wl.qo_indptr, wl.kv_indptr, d["kv_indices"], wl.last_page_len, 8, 2, 128,
                      16, causal=False)
    out, lse = ak.ak_run(plan, d["q"], d["k_cache"], d["v_cache"],
                         lse=torch.empty(T, 8, device="cuda"))
    torch.cuda.synchronize()
    empty = slice(int(wl.qo_indptr[1]), int(wl.qo_indptr[2]))
    assert torch.all(out[empty].float() == 0) and torch.all(torch.isneginf(lse[empty]))
    keep = [0, 2]
    from gpu_harness import compare
    eo, el, n = compare(wl, out, lse, -1, requests=keep)
    say(f"  rows={n} max|dout|={eo:.3e} max|dlse|={el:.3e}")
    assert eo <= TOL["bf16"][0] and el <= TOL["bf16"][1]


def test_cascade_segments_on_two_streams():
    # the shared segment on a side stream beside the suffix decode on the main
    # stream, joined by an event before the merge: the same result
    R, B, hq, hkv, D, k = 16, 16, 32, 8, 128, 32
    rng = np.random.default_rng(5)
    kl = rng.integers(k * B + 2, k * B + 900, size=R)
    wl = W.custom(seed=41, q_lens=np.ones(R, np.int64), kv_lens=kl, page_size=B, num_qo_heads=hq,
                  num_kv_heads=hkv, head_dim=D, name="cascade_2s")
    for r in range(1, R):
        wl.kv_indices[wl.kv_indptr[r]:wl.kv_indptr[r] + k] = wl.kv_indices[:k]
    d = prepare(wl)
    T = wl.total_q
    shared = ak.ak_plan([0, T], [0, k], torch.from_numpy(wl.kv_indices[:k].copy()).cuda(), [B],
                        hq, hkv, D, B, causal=False)
    sx = np.concatenate([wl.kv_indices[wl.kv_indptr[r] + k:wl.kv_indptr[r + 1]] for r in range(R)])
    si = np.concatenate([[0], np.cumsum(np.diff(wl.kv_indptr) - k)]).astype(np.int32)
    suffix = ak.ak_plan(wl.qo_indptr, si, torch.from_numpy(sx.astype(np.int32)).cuda(),
                        wl.last_page_len, hq, hkv, D, B)
    side, main = torch.cuda.Stream(), torch.cuda.current_stream()
    o1 = torch.empty_like(d["q"])
    l1 = torch.empty(T, hq, device="cuda")
    start = torch.cuda.Event()
    start.record(main)
    side.wait_event(start)
    ak.ak_run(shared, d["q"], d["k_cache"], d["v_cache"], out=o1, lse=l1, stream=side)
    done = torch.cuda.Event()
    done.record(side)
    o2, l2 = ak.ak_run(suffix, d["q"], d["k_cache"], d["v_cache"], lse=torch.empty(T, hq, device="cuda"))
    main.wait_event(done)
    out, lse = ak.ak_merge_states(o1, l1, o2, l2)
    torch.cuda.synchronize()
    check(wl, out, lse, -1)
