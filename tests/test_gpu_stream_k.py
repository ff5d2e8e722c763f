"""Stream-K decode plans (AK_PLAN_STREAM_K) on the GPU against the fp64 CPU
oracle: persistent workgroups each running the pieces of one equal share of the
decode units' KV, units cut across shares merged from partial states.  Reduced
workloads compared in full, the full-size decode and long fp8 decode on sampled
rows, and edge cases; few compute units in the plan force many pieces per
workgroup (the persistent loop), the in-kernel merge is exercised too, and
repeated runs are bitwise identical."""

import numpy as np
import pytest
import torch

import paged_kv_attention_store_amd as ak
from synth import workloads as W
from tests.gpu_harness import check, plan_for, prepare, run, say
from tests.test_gpu_parity import _full_size_requests, _sample_rows

pytestmark = pytest.mark.gpu

VARIANTS = [{}, {"num_cus": 4}, {"merge_in_kernel": True}, {"num_cus": 16, "merge_in_kernel": True}]
VARIANT_IDS = ["default", "4cus", "merge_in_kernel", "16cus_merge_in_kernel"]


def _run_all(wl, windows=None, **kw):
    d = prepare(wl)
    for window in (windows or wl.windows):
        plan = plan_for(wl, d, window, stream_k=True, **kw)
        info = ak.ak_plan_info(plan)
        say(f"[stream-k] {wl.name} window={window} {kw} workgroups={info['stream_k_workgroups']} "
            f"items={info['small_items']} split_units={info['split_units']}")
        out, lse = run(wl, d, plan)
        check(wl, out, lse, window)
        out2, lse2 = run(wl, d, plan)
        assert torch.equal(out, out2) and torch.equal(lse, lse2), "runs differ"


@pytest.mark.parametrize("kw", VARIANTS, ids=VARIANT_IDS)
def test_stream_k_decode_reduced(kw):
    _run_all(W.llama8b_decode(seed=2, R=8), **kw)


@pytest.mark.parametrize("kw", VARIANTS, ids=VARIANT_IDS)
def test_stream_k_mixed_reduced(kw):
    wl = W.mixed_chunk_decode(seed=4, R_dec=40, chunk=300, prefix=700, lmin=100, lmax=6000)
    _run_all(wl, windows=(-1, 4096, 256), **kw)


@pytest.mark.parametrize("kw", VARIANTS[:2], ids=VARIANT_IDS[:2])
def test_stream_k_long_decode_fp8_reduced(kw):
    _run_all(W.llama70b_long_decode(seed=5, R=2, L=20000), **kw)


def test_stream_k_tiny_fp32():
    _run_all(W.config(1), num_cus=1)


EDGE = [
    # name, q_lens, kv_lens, B, hq, hkv, D, kv_dtype, windows
    ("page_size_1_long", [1, 1, 2], [5000, 3000, 2049], 1, 8, 2, 128, "bf16", (-1, 700)),
    ("gqa_g16", [1, 1, 1], [700, 65, 3000], 16, 32, 2, 128, "bf16", (-1, 50)),
    ("head_dim_64", [1, 2, 1], [333, 2600, 64], 16, 16, 4, 64, "bf16", (-1, 20)),
    ("head_dim_64_fp8", [1, 2, 1], [333, 2600, 64], 16, 16, 4, 64, "fp8", (-1, 20)),
    ("fp8_g8_pages64", [1, 1], [9000, 130], 64, 64, 8, 128, "fp8", (-1, 1000)),
    ("one_key", [1, 1, 1], [1, 2, 17], 16, 8, 2, 128, "bf16", (-1, 0)),
]


@pytest.mark.parametrize("case", EDGE, ids=[c[0] for c in EDGE])
def test_stream_k_edge_cases(case):
    name, ql, kl, B, hq, hkv, D, kd, windows = case
    wl = W.custom(seed=len(name) * 17 + sum(kl), q_lens=ql, kv_lens=kl, page_size=B,
                  num_qo_heads=hq, num_kv_heads=hkv, head_dim=D, kv_dtype=kd, windows=windows,
                  name=f"streamk_{name}")
    for kw in ({"num_cus": 2}, {"num_cus": 64}, {"num_cus": 3, "merge_in_kernel": True}):
        _run_all(wl, **kw)


@pytest.mark.parametrize("k", [2, 4, 5])
def test_stream_k_full_size_sampled(k):
    wl = W.config(k)
    d = prepare(wl)
    reqs = _full_size_requests(wl, k)
    for window in wl.windows:
        plan = plan_for(wl, d, window, stream_k=True)
        say(f"[stream-k full] config {k} window={window} {ak.ak_plan_info(plan)}")
        out, lse = run(wl, d, plan)
        check(wl, out, lse, window, requests=reqs,
              rows_of=lambda r, w=window: _sample_rows(wl, r, window=w))
    del d
    torch.cuda.empty_cache()
