"""Split decode merged inside the attention kernel (plan flag
AK_PLAN_MERGE_IN_KERNEL), GPU vs oracle and vs the separate merge launch.

The parts of a split (request, KV head) unit combine their states by the
log-sum-exp rule ("SGLang attention backend", "The two forms of extend"); with
the flag the last part to finish does it.  Whichever workgroup that is, the
parts are combined in part order, so repeated runs are bit-identical, and the
arithmetic is the merge kernel's, so the two paths agree.
"""

import numpy as np
import pytest
import torch

import paged_kv_attention_store_amd as ak
from synth import rng as R
from synth import workloads as W

from gpu_harness import check, plan_for, prepare, run, say

pytestmark = pytest.mark.gpu

BF16_ULP_REL = 2.0 ** -8


def _agree(a, b):
    """Two bf16 outputs within one bf16 ulp of each other (same arithmetic, at most
    a contraction difference in fp32)."""
    a, b = a.float(), b.float()
    return bool(torch.all((a - b).abs() <= BF16_ULP_REL * torch.maximum(a.abs(), b.abs()) + 1e-30))


CASES = [
    # name, workload factory, plan options
    ("decode_d128", lambda: W.llama8b_decode(seed=2, R=8), dict(min_chunk=64)),
    ("decode_many_parts", lambda: W.llama8b_decode(seed=7, R=6), dict(min_chunk=64, num_cus=512)),
    ("decode_d64_g8", lambda: W.custom(seed=9, q_lens=[1, 1, 2, 1], kv_lens=[3000, 700, 1900, 65],
                                       page_size=16, num_qo_heads=16, num_kv_heads=2, head_dim=64,
                                       name="d64_g8"), dict(min_chunk=64)),
    ("fp8_long", lambda: W.llama70b_long_decode(seed=5, R=2, L=20000), {}),
    ("mixed", lambda: W.mixed_chunk_decode(seed=4, R_dec=40, chunk=300, prefix=700, lmin=100,
                                           lmax=6000), dict(min_chunk=64)),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_merge_in_kernel_matches_oracle_and_merge_launch(case):
    name, make, kw = case
    wl = make()
    d = prepare(wl)
    fused = plan_for(wl, d, wl.windows[0], merge_in_kernel=True, **kw)
    plain = plan_for(wl, d, wl.windows[0], **kw)
    info = ak.ak_plan_info(fused)
    say(f"[merge-in-kernel] {name}: {info}")
    assert info["split_units"] > 0
    o1, l1 = run(wl, d, fused)
    o2, l2 = run(wl, d, fused)
    # the merging workgroup differs from run to run; the bits do not
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    o3, l3 = run(wl, d, plain)
    assert _agree(o1, o3)
    assert float((l1 - l3).abs().max()) <= 1e-5
    check(wl, o1, l1, wl.windows[0])


def test_merge_in_kernel_across_layers_resets_counters():
    # the arrival counters return to zero after every run: many runs of one plan
    # with fresh queries stay correct
    wl = W.llama8b_decode(seed=2, R=8)
    d = prepare(wl)
    plan = plan_for(wl, d, -1, min_chunk=64, merge_in_kernel=True)
    plain = plan_for(wl, d, -1, min_chunk=64)
    for layer in range(6):
        q = torch.empty_like(d["q"])
        R.fill_torch(q, 200 + layer, "q")
        o1, l1 = run(wl, d, plan, q=q)
        o2, l2 = run(wl, d, plain, q=q)
        assert _agree(o1, o2), f"layer {layer}"
        assert float((l1 - l2).abs().max()) <= 1e-5


@pytest.mark.parametrize("stream_k", [False, True], ids=["split_kv", "stream_k"])
def test_merge_in_kernel_publication_back_to_back(stream_k):
    # The merging workgroup reads the other parts' partial rows after counting
    # itself in; a part whose rows were not yet visible would hand it the previous
    # run's rows.  Runs alternate two query sets and are enqueued back to back
    # without a host synchronisation, so the partial buffers always hold the
    # other query set's rows from the run before: every run must still equal the
    # separate merge launch on its own queries.
    wl = W.llama8b_decode(seed=7, R=12)
    d = prepare(wl)
    kw = dict(stream_k=True, num_cus=64) if stream_k else dict(min_chunk=64, num_cus=512)
    fused = plan_for(wl, d, -1, merge_in_kernel=True, **kw)
    plain = plan_for(wl, d, -1, **kw)
    info = ak.ak_plan_info(fused)
    say(f"[merge-in-kernel] back-to-back, {info}")
    assert info["split_units"] > 0
    qs = []
    for s in (300, 301):
        q = torch.empty_like(d["q"])
        R.fill_torch(q, s, "q")
        qs.append(q)
    refs = [run(wl, d, plain, q=q) for q in qs]
    outs = []
    for i in range(40):
        q = qs[i % 2]
        o = torch.empty_like(q)
        lse = torch.empty(wl.total_q, wl.num_qo_heads, dtype=torch.float32, device=q.device)
        ak.ak_run(fused, q, d["k_cache"], d["v_cache"], out=o, lse=lse)
        outs.append((o, lse))
    torch.cuda.synchronize()
    for i, (o, lse) in enumerate(outs):
        ro, rl = refs[i % 2]
        assert _agree(o, ro), f"run {i}"
        assert float((lse - rl).abs().max()) <= 1e-5, f"run {i}"
