"""Device-side batch metadata (GPU vs oracle, bit-exact):

* ak_csr_from_block_table against the oracle's block table -> CSR rewrite
  ("vLLM attention backend", "From a 2-D block table to a CSR page table"),
  on the page's worked example and on random batches with empty requests, full
  last pages, padded rows and batches larger than one scan chunk;
* ak_slot_mapping against the oracle's slot arithmetic ("Write the KV first" and
  the worked example), with padding tokens past the batch;
* one step driven from a block table alone: device CSR and slots feed
  ak_store_kv, ak_plan and ak_run, and the output matches the oracle.
"""

import json
import pathlib

import numpy as np
import pytest
import torch

import paged_kv_attention_store_amd as ak
from oracle import metadata as M
from synth import workloads as W

from gpu_harness import check, plan_for, prepare, run, say

pytestmark = pytest.mark.gpu

GOLDEN = pathlib.Path(__file__).parent / "golden"
JUNK = -123456   # padding past a row's valid pages: must never reach the output


def _table(rows, max_pages, rng=None):
    t = np.full((len(rows), max_pages), JUNK, dtype=np.int32)
    if rng is not None:
        t[:] = rng.integers(-(1 << 30), 1 << 30, size=t.shape)
    for r, row in enumerate(rows):
        t[r, :len(row)] = row
    return t


def _new_positions(seq_lens, q_lens):
    return [list(range(int(L) - int(n), int(L))) for L, n in zip(seq_lens, q_lens)]


def _device_csr(table, seq_lens, B, capacity=None, fill=-7):
    bt = torch.from_numpy(table).cuda()
    sl = torch.from_numpy(np.asarray(seq_lens, np.int32)).cuda()
    R, mp = table.shape
    cap = R * mp if capacity is None else capacity
    idx = torch.full((max(cap, 1),), fill, dtype=torch.int32, device="cuda")[:cap]
    ip, ix, lp = ak.ak_csr_from_block_table(bt, sl, B, kv_indices=idx)
    torch.cuda.synchronize()
    return ip.cpu().numpy(), ix.cpu().numpy(), lp.cpu().numpy()


def test_worked_example():
    g = json.loads((GOLDEN / "vllm_worked_example.json").read_text())
    B, e = g["page_size"], g["expect"]
    table = _table(g["block_rows"], 8)
    ip, ix, lp = _device_csr(table, g["seq_lens"], B)
    n = ip[-1]
    assert ip.tolist() == e["paged_kv_indptr"]
    assert ix[:n].tolist() == e["paged_kv_indices"]
    assert lp.tolist() == e["paged_kv_last_page_len"]
    qo = torch.tensor(g["query_start_loc"], dtype=torch.int32, device="cuda")
    slots = ak.ak_slot_mapping(torch.from_numpy(table).cuda(), qo,
                               torch.tensor(g["seq_lens"], dtype=torch.int32, device="cuda"), B)
    assert slots.cpu().tolist() == e["slot_mapping"]


@pytest.mark.parametrize("R,B,max_pages,seed", [
    (1, 16, 4, 0),
    (37, 16, 70, 1),
    (300, 1, 40, 2),
    (1500, 64, 33, 3),      # more than one 1024-request chunk of the running sum
    (4096, 16, 9, 4),
])
def test_csr_and_slots_bit_exact(R, B, max_pages, seed):
    rng = np.random.default_rng(seed)
    L = rng.integers(0, max_pages * B + 1, size=R)
    L[rng.random(R) < 0.1] = 0                                   # empty requests
    full = rng.random(R) < 0.1
    L[full] = (L[full] // B) * B                                 # full last pages
    L[-1] = max_pages * B                                        # a full row
    rows = [rng.integers(0, 1 << 20, size=-(-int(l) // B)) for l in L]
    table = _table(rows, max_pages, rng)
    say(f"[metadata] R={R} B={B} max_pages={max_pages} pages={sum(len(r) for r in rows)}")
    ip, ix, lp = _device_csr(table, L, B)
    ei, ex, el = M.block_table_to_csr(L, rows, B)
    assert np.array_equal(ip, ei)
    assert np.array_equal(ix[:ip[-1]], ex)
    assert np.array_equal(lp, el)
    # this step's tokens: n_r in [0, min(L_r, 40)], then padding tokens past the batch
    n = np.minimum(rng.integers(0, 41, size=R), L)
    qo = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    pad = 131
    out = torch.full((int(qo[-1]) + pad,), -7, dtype=torch.int64, device="cuda")
    ak.ak_slot_mapping(torch.from_numpy(table).cuda(), torch.from_numpy(qo).cuda(),
                       torch.from_numpy(L.astype(np.int32)).cuda(), B, out=out)
    got = out.cpu().numpy()
    exp = M.slot_mapping(rows, _new_positions(L, n), B)
    assert np.array_equal(got[:qo[-1]], exp)
    assert np.all(got[qo[-1]:] == -1)


@pytest.mark.parametrize("ratio,B", [(2, 16), (4, 16), (8, 8), (3, 32)])
def test_csr_virtual_blocks_bit_exact(ratio, B):
    rng = np.random.default_rng(ratio * B)
    R, mb = 300, 20
    Mtok = ratio * B
    L = rng.integers(0, mb * Mtok + 1, size=R)
    L[::17] = 0
    L[5] = mb * Mtok
    rows = [rng.integers(0, 5000, size=-(-int(l) // Mtok)) for l in L]
    table = _table(rows, mb, rng)
    bt = torch.from_numpy(table).cuda()
    ip, ix, lp = ak.ak_csr_from_block_table(bt, torch.from_numpy(L.astype(np.int32)).cuda(), B,
                                            block_ratio=ratio)
    torch.cuda.synchronize()
    ip, ix, lp = ip.cpu().numpy(), ix.cpu().numpy(), lp.cpu().numpy()
    ei, ex, el = M.block_table_to_csr(L, M.virtual_block_rows(rows, ratio), B)
    assert np.array_equal(ip, ei) and np.array_equal(ix[:ip[-1]], ex) and np.array_equal(lp, el)


def test_attention_through_virtual_kernel_blocks():
    # the cache is managed in 64-token blocks; the kernels read it as 16-token pages
    wl = W.custom(seed=41, q_lens=[1, 1, 20, 1], kv_lens=[700, 64, 300, 1], page_size=64,
                  num_qo_heads=32, num_kv_heads=8, head_dim=128, name="virtual_blocks")
    say("[metadata] 64-token manager blocks as 16-token kernel pages")
    d = prepare(wl)
    ratio, B = 4, 16
    table = _table(wl.req_pages, max(len(p) for p in wl.req_pages))
    sl = torch.from_numpy(wl.kv_lens.astype(np.int32)).cuda()
    ip, ix, lp = ak.ak_csr_from_block_table(torch.from_numpy(table).cuda(), sl, B, block_ratio=ratio)
    P = wl.num_pages
    kc = d["k_cache"].view(P * ratio, B, 8, 128)
    vc = d["v_cache"].view(P * ratio, B, 8, 128)
    plan = ak.ak_plan(wl.qo_indptr, ip.cpu().numpy(), ix, lp.cpu().numpy(), 32, 8, 128, B)
    out, lse = ak.ak_run(plan, d["q"], kc, vc, lse=torch.empty(wl.total_q, 32, device="cuda"))
    torch.cuda.synchronize()
    check(wl, out, lse, -1)


def test_csr_capacity_and_clamped_lengths():
    rng = np.random.default_rng(11)
    R, B, mp = 50, 16, 6
    L = rng.integers(1, mp * B + 1, size=R)
    rows = [rng.integers(0, 1000, size=mp) for _ in range(R)]
    table = _table(rows, mp)
    ei, ex, el = M.block_table_to_csr(L, rows, B)
    cap = int(ei[-1]) // 2
    ip, ix, lp = _device_csr(table, L, B, capacity=cap)
    assert np.array_equal(ip, ei) and np.array_equal(lp, el)
    assert np.array_equal(ix, ex[:cap])                 # nothing written past capacity
    # lengths beyond the row and negative lengths are clamped to [0, mp * B]
    Lc = L.copy()
    Lc[::3] = mp * B + 1000
    Lc[1::7] = -5
    ip, ix, lp = _device_csr(table, Lc, B)
    ei, ex, el = M.block_table_to_csr(np.clip(Lc, 0, mp * B), rows, B)
    assert np.array_equal(ip, ei) and np.array_equal(ix[:ip[-1]], ex) and np.array_equal(lp, el)


def test_metadata_rejects_bad_arguments():
    bt = torch.zeros(2, 3, dtype=torch.int32, device="cuda")
    sl = torch.ones(2, dtype=torch.int32, device="cuda")
    with pytest.raises(ak.AkError) as e:
        ak.ak_csr_from_block_table(bt, sl, 0)
    assert e.value.status == ak.AK_ERR_INVALID_ARG
    with pytest.raises(ak.AkError):
        ak.ak_csr_from_block_table(bt.long(), sl, 16)
    with pytest.raises(ak.AkError) as e:
        ak.ak_slot_mapping(bt, torch.zeros(3, dtype=torch.int32, device="cuda"), sl, -1,
                           num_tokens=4)
    assert e.value.status == ak.AK_ERR_INVALID_ARG
    # an empty batch: kv_indptr = [0], nothing else touched
    ip, ix, lp = ak.ak_csr_from_block_table(torch.zeros(0, 4, dtype=torch.int32, device="cuda"),
                                            torch.zeros(0, dtype=torch.int32, device="cuda"), 16)
    assert ip.cpu().tolist() == [0]


def _mixed():
    return W.custom(seed=21, q_lens=[1, 1, 37, 1, 200, 5], kv_lens=[33, 900, 37, 1, 700, 64],
                    page_size=16, num_qo_heads=32, num_kv_heads=8, head_dim=128, name="mixed_meta")


@pytest.mark.parametrize("k", [1, 0])
def test_step_from_block_table(k):
    wl = W.config(k) if k else _mixed()
    B = wl.page_size
    mp = max(len(p) for p in wl.req_pages) + 3
    table = _table(wl.req_pages, mp, np.random.default_rng(k))
    say(f"[metadata step] {wl.name}")
    d = prepare(wl, store_new=False)
    bt = torch.from_numpy(table).cuda()
    sl = torch.from_numpy(wl.kv_lens.astype(np.int32)).cuda()
    qo = torch.from_numpy(wl.qo_indptr.astype(np.int32)).cuda()
    ip, ix, lp = ak.ak_csr_from_block_table(bt, sl, B)
    slots = ak.ak_slot_mapping(bt, qo, sl, B, num_tokens=wl.total_q)
    ak.ak_store_kv(d["k_new"], d["v_new"], slots, d["k_cache"], d["v_cache"], wl.kv_scale,
                   wl.kv_scale)
    # the plan reads the host copies of the lengths; the page ids stay on the device
    assert np.array_equal(ip.cpu().numpy(), wl.kv_indptr)
    assert np.array_equal(lp.cpu().numpy(), wl.last_page_len)
    plan = plan_for(wl, {"kv_indices": ix}, wl.windows[0])
    out, lse = run(wl, d, plan)
    check(wl, out, lse, wl.windows[0])
