"""The plan's KV indexing on the GPU, bit-exact against the oracle's slot
arithmetic, and the exported work list of every workload."""

import numpy as np
import pytest
import torch

import paged_kv_attention_store_amd as ak
from oracle import metadata as M
from synth import workloads as W
from tests.gpu_harness import plan_for, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("addressing", [0, 1, 2], ids=["decode_rows", "prefill_copies",
                                                      "prefill_copies32"])
@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
def test_gather_slots_bit_exact(k, addressing):
    # the slots come from the kernels' own K/V addressing functions (page-id read,
    # clamp, row offset) run with page stride B and slot stride 1
    say(f"[indexing] config {k}, addressing {addressing}")
    wl = W.config(k)
    idx = torch.from_numpy(wl.kv_indices.astype(np.int32)).cuda()
    plan = plan_for(wl, {"kv_indices": idx}, wl.windows[0])
    total = int(wl.kv_lens.sum())
    slots = torch.full((total,), -7, dtype=torch.int64, device="cuda")
    ak.ak_gather_slots(plan, slots, addressing=addressing)
    got = slots.cpu().numpy()
    exp = np.concatenate([M.request_slots(wl.kv_indptr, wl.kv_indices, wl.last_page_len,
                                          wl.page_size, r) for r in range(wl.batch_size)])
    assert np.array_equal(got, exp)
    items, lens = ak.ak_plan_export(plan)
    assert lens.tolist() == M.kv_lengths(wl.kv_indptr, wl.last_page_len, wl.page_size).tolist()


INDEX_EDGE = [
    # name, q_lens, kv_lens, page size
    ("page_256", [1, 3, 1], [1000, 513, 256], 256),
    ("page_2", [1, 1, 2], [5, 4097, 2], 2),
    ("no_pages", [1, 0, 1], [77, 0, 1], 16),
]


@pytest.mark.parametrize("addressing", [0, 1, 2], ids=["decode_rows", "prefill_copies",
                                                      "prefill_copies32"])
@pytest.mark.parametrize("case", INDEX_EDGE, ids=[c[0] for c in INDEX_EDGE])
def test_gather_slots_edge_geometries(case, addressing):
    name, ql, kl, B = case
    wl = W.custom(seed=61 + B, q_lens=ql, kv_lens=kl, page_size=B, num_qo_heads=8,
                  num_kv_heads=2, head_dim=128, name=name)
    idx = torch.from_numpy(wl.kv_indices.astype(np.int32)).cuda()
    plan = plan_for(wl, {"kv_indices": idx}, -1)
    total = int(wl.kv_lens.sum())
    slots = torch.full((total,), -7, dtype=torch.int64, device="cuda")
    ak.ak_gather_slots(plan, slots, addressing=addressing)
    exp = np.concatenate([M.request_slots(wl.kv_indptr, wl.kv_indices, wl.last_page_len,
                                          wl.page_size, r) for r in range(wl.batch_size)])
    assert np.array_equal(slots.cpu().numpy(), exp)
