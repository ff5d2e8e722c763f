"""A whole step captured once into a HIP graph and replayed over changing
batches (GPU vs eager runs and vs the oracle).

The captured step is: block table -> CSR page table (ak_csr_from_block_table),
slot of every new token (ak_slot_mapping), the store of this step's K/V
(ak_store_kv) and attention with a fixed plan (ak_run).  Every buffer the graph
touches has a fixed address and is sized for the largest batch; between replays
the host writes the next batch's contents into those buffers and updates the
fixed plan ("vLLM attention backend", graph-capture section; "SGLang attention
backend", the backend's graph duties).  Padding requests have no tokens and no
pages, and padding tokens get slot -1, which the store skips.

Each replay must equal, bit for bit, an eager run of an ordinary plan over the
same cache, and match the oracle within the bf16 bound.
"""

import numpy as np
import pytest
import torch

import paged_kv_attention_store_amd as ak
from synth import workloads as W

from gpu_harness import check, prepare, say

pytestmark = pytest.mark.gpu

HQ, HKV, D, B = 32, 8, 128, 16
R_MAX, T_MAX, ROW_PAGES = 48, 288, 200
BATCHES = [
    # (seed, q_lens, kv_lens)
    (31, [1] * 40, list(np.linspace(100, 3000, 40).astype(int))),
    (32, [1] * 10 + [37, 200], [900, 17, 64, 1500, 3000, 1, 250, 777, 2048, 16, 300, 2600]),
    (33, [1, 1, 5], [3000, 40, 2999]),
    (34, [1] * 48, [2900 - 50 * i for i in range(48)]),
    (35, [1] * 40, list(np.linspace(100, 3000, 40).astype(int))),   # first batch again
]


def _random_batch(seed):
    """A seeded batch within the captured capacities: 1 to 48 requests, mostly
    decodes, some 2-5 token queries and 6-64 token extend chunks, KV lengths up
    to a table row's 200 pages."""
    rng = np.random.default_rng(seed)
    q = []
    for _ in range(int(rng.integers(1, R_MAX + 1))):
        u = rng.random()
        q.append(1 if u < 0.75 else int(rng.integers(2, 6)) if u < 0.9 else int(rng.integers(6, 65)))
    while sum(q) > T_MAX:
        q[int(np.argmax(q))] //= 2
    kv = [int(rng.integers(qi, ROW_PAGES * B + 1)) for qi in q]
    return (seed, q, kv)


BATCHES += [_random_batch(s) for s in (36, 37, 38)]


def _workload(seed, q_lens, kv_lens):
    return W.custom(seed=seed, q_lens=q_lens, kv_lens=kv_lens, page_size=B, num_qo_heads=HQ,
                    num_kv_heads=HKV, head_dim=D, name=f"graph_{seed}")


@pytest.mark.parametrize("merge_in_kernel", [False, True], ids=["merge_launch", "merge_in_kernel"])
def test_captured_step_replays_every_batch(merge_in_kernel):
    wls = [_workload(*b) for b in BATCHES]
    P = max(wl.num_pages for wl in wls)
    dev = "cuda"
    # fixed-address buffers, sized for the largest batch
    k_cache = torch.zeros(P, B, HKV, D, dtype=torch.bfloat16, device=dev)
    v_cache = torch.zeros_like(k_cache)
    table = torch.zeros(R_MAX, ROW_PAGES, dtype=torch.int32, device=dev)
    seq_lens = torch.zeros(R_MAX, dtype=torch.int32, device=dev)
    qo_dev = torch.zeros(R_MAX + 1, dtype=torch.int32, device=dev)
    kv_indptr = torch.zeros(R_MAX + 1, dtype=torch.int32, device=dev)
    last = torch.zeros(R_MAX, dtype=torch.int32, device=dev)
    kv_indices = torch.zeros(R_MAX * ROW_PAGES, dtype=torch.int32, device=dev)
    slots = torch.zeros(T_MAX, dtype=torch.int64, device=dev)
    q = torch.zeros(T_MAX, HQ, D, dtype=torch.bfloat16, device=dev)
    k_new = torch.zeros(T_MAX, HKV, D, dtype=torch.bfloat16, device=dev)
    v_new = torch.zeros_like(k_new)
    out = torch.zeros(T_MAX, HQ, D, dtype=torch.bfloat16, device=dev)
    lse = torch.zeros(T_MAX, HQ, dtype=torch.float32, device=dev)
    plan = ak.ak_plan_fixed(R_MAX, T_MAX, kv_indices, HQ, HKV, D, B, merge_in_kernel=merge_in_kernel)
    info = plan.info()
    say(f"[graph] capacities small={info['cap_small_items']} large={info['cap_large_items']} "
        f"merges={info['cap_merge_jobs']} partial_rows={info['cap_partial_rows']}")

    def load(wl):
        """Write one batch into the fixed buffers (eager work between replays)."""
        d = prepare(wl, store_new=False)
        R, T = wl.batch_size, wl.total_q
        k_cache[:wl.num_pages].copy_(d["k_cache"])
        v_cache[:wl.num_pages].copy_(d["v_cache"])
        tb = np.full((R_MAX, ROW_PAGES), -99, np.int32)
        for r, pages in enumerate(wl.req_pages):
            tb[r, :len(pages)] = pages
        sl = np.zeros(R_MAX, np.int32)
        sl[:R] = wl.kv_lens
        qo = np.full(R_MAX + 1, T, np.int32)
        qo[:R + 1] = wl.qo_indptr
        table.copy_(torch.from_numpy(tb))
        seq_lens.copy_(torch.from_numpy(sl))
        qo_dev.copy_(torch.from_numpy(qo))
        q[:T].copy_(d["q"])
        k_new[:T].copy_(d["k_new"])
        v_new[:T].copy_(d["v_new"])
        ak.ak_plan_update(plan, wl.qo_indptr, wl.kv_indptr, wl.last_page_len)
        return d

    def step():
        ak.ak_csr_from_block_table(table, seq_lens, B, kv_indices=kv_indices, kv_indptr=kv_indptr,
                                   last_page_len=last)
        ak.ak_slot_mapping(table, qo_dev, seq_lens, B, out=slots)
        ak.ak_store_kv(k_new, v_new, slots, k_cache, v_cache)
        ak.ak_run(plan, q, k_cache, v_cache, out=out, lse=lse)

    load(wls[0])
    step()                                   # eager warm-up (loads every kernel)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i, wl in enumerate(wls):
        T = wl.total_q
        d = load(wl)
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        say(f"[graph] replay {i}: R={wl.batch_size} T={T} items={plan.info()['items']}")
        # the device-built metadata is the batch's own
        assert np.array_equal(kv_indptr[:wl.batch_size + 1].cpu().numpy(), wl.kv_indptr)
        assert np.array_equal(slots[:T].cpu().numpy(), wl.slot_mapping)
        assert torch.all(slots[T:] == -1)
        o1, l1 = out[:T].clone(), lse[:T].clone()
        g.replay()                           # the store is idempotent: same result again
        torch.cuda.synchronize()
        assert torch.equal(out[:T], o1) and torch.equal(lse[:T], l1)
        # an eager ordinary plan over the same (stored) cache gives the same bits
        ref = ak.ak_plan(wl.qo_indptr, wl.kv_indptr, d["kv_indices"], wl.last_page_len, HQ, HKV,
                         D, B, merge_in_kernel=merge_in_kernel)
        eo = torch.empty(T, HQ, D, dtype=torch.bfloat16, device=dev)
        el = torch.empty(T, HQ, dtype=torch.float32, device=dev)
        ak.ak_run(ref, q[:T], k_cache, v_cache, out=eo, lse=el)
        torch.cuda.synchronize()
        assert torch.equal(eo, o1) and torch.equal(el, l1)
        check(wl, o1, l1, -1)


@pytest.mark.filterwarnings("ignore:The CUDA Graph is empty")
def test_plan_calls_refused_inside_capture():
    # creating or updating a fixed plan synchronises and copies from the host:
    # inside a capture both are refused with a clear error (and nothing is recorded)
    kv_indices = torch.zeros(64, dtype=torch.int32, device="cuda")
    plan = ak.ak_plan_fixed(4, 8, kv_indices, HQ, HKV, D, B)
    g = torch.cuda.CUDAGraph()
    errors = []
    with torch.cuda.graph(g):
        for call in (lambda: ak.ak_plan_fixed(4, 8, kv_indices, HQ, HKV, D, B),
                     lambda: ak.ak_plan_update(plan, [0, 1], [0, 1], [5])):
            try:
                call()
            except ak.AkError as e:
                errors.append((e.status, ak.ak_last_error()))
    assert [s for s, _ in errors] == [ak.AK_ERR_INVALID_ARG] * 2
    assert all("captured" in m for _, m in errors)
    ak.ak_plan_update(plan, [0, 1], [0, 1], [5])      # outside the capture: fine
