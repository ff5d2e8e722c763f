"""ak_run_noalloc (plan + run with the split workspace in the library's fixed
device array) against ak_plan + ak_run on the same inputs, through the C ABI:
two calls in a row, the second on a smaller batch, each bit-identical to the
allocating entry points and within the oracle's tolerances; the arrival
counters of the in-kernel merge start from zero on every call; a batch too
large for the array is refused before anything is enqueued."""

import ctypes

import numpy as np
import pytest
import torch

import paged_kv_attention_store_amd as ak
from synth import workloads as W
from tests.gpu_harness import check, plan_for, prepare, run, say

pytestmark = pytest.mark.gpu


def _noalloc(wl, d, window, **kw):
    out = torch.full_like(d["q"], float("nan"))
    lse = torch.full((wl.total_q, wl.num_qo_heads), float("nan"), dtype=torch.float32,
                     device=d["q"].device)
    ak.ak_run_noalloc(wl.qo_indptr, wl.kv_indptr, d["kv_indices"], wl.last_page_len,
                      wl.num_qo_heads, wl.num_kv_heads, wl.head_dim, wl.page_size, d["q"],
                      d["k_cache"], d["v_cache"], out, lse, causal=wl.causal, window=window,
                      k_scale=wl.kv_scale, v_scale=wl.kv_scale, **kw)
    torch.cuda.synchronize()
    return out, lse


def _same_as_plan_and_run(wl, d, window, **kw):
    out, lse = _noalloc(wl, d, window, **kw)
    ref_out, ref_lse = run(wl, d, plan_for(wl, d, window, **kw))
    assert torch.equal(out, ref_out), "out differs from ak_plan + ak_run"
    assert torch.equal(lse, ref_lse), "lse differs from ak_plan + ak_run"
    check(wl, out, lse, window)


@pytest.mark.parametrize("merge_in_kernel", [False, True])
def test_noalloc_equals_plan_and_run_two_calls(merge_in_kernel):
    kw = {"merge_in_kernel": merge_in_kernel}
    # first call: a mixed batch (large tiles, small tiles, split decode units)
    big = W.mixed_chunk_decode(seed=4, R_dec=40, chunk=300, prefix=700, lmin=100, lmax=6000)
    say(f"[noalloc] call 1: {big.name} R={big.batch_size} tokens={big.total_q} "
        f"merge_in_kernel={merge_in_kernel}")
    d = prepare(big)
    for window in (-1, 256):
        _same_as_plan_and_run(big, d, window, **kw)
    del d
    # second call: a smaller decode batch, forced to split (fewer items, fewer
    # partial rows and counters than the first left in the array)
    small = W.llama8b_decode(seed=7, R=6)
    say(f"[noalloc] call 2: {small.name} R={small.batch_size}")
    d = prepare(small)
    _same_as_plan_and_run(small, d, -1, min_chunk=64, num_cus=512, **kw)


def test_noalloc_stream_k():
    # a stream-K plan's workgroup table travels in the same array
    wl = W.llama8b_decode(seed=2, R=8)
    say(f"[noalloc] stream-K {wl.name}")
    d = prepare(wl)
    _same_as_plan_and_run(wl, d, -1, stream_k=True, num_cus=16)
    _same_as_plan_and_run(wl, d, -1, stream_k=True, merge_in_kernel=True)


def test_noalloc_fp8_and_fp32():
    for wl in (W.llama70b_long_decode(seed=5, R=2, L=20000), W.config(1)):
        say(f"[noalloc] {wl.name}")
        d = prepare(wl)
        _same_as_plan_and_run(wl, d, -1)


def test_noalloc_refuses_a_batch_beyond_the_array():
    # 512 decodes of 32768 tokens at 64/8 heads: about 137 MiB of work list and
    # split partials, refused on the host (tiny tensors: nothing is launched)
    R, L, B = 512, 32768, 16
    qo = np.arange(R + 1, dtype=np.int32)
    kv = np.arange(R + 1, dtype=np.int32) * (L // B)
    last = np.full(R, B, dtype=np.int32)
    idx = torch.zeros(1, dtype=torch.int32, device="cuda")
    q = torch.zeros(R, 64, 128, dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros(1, B, 8, 128, dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q)
    with pytest.raises(ak.AkError) as e:
        ak.ak_run_noalloc(qo, kv, idx, last, 64, 8, 128, B, q, kc, kc, out)
    assert e.value.status == ak.AK_ERR_UNSUPPORTED and "scratch" in ak.ak_last_error()


def test_noalloc_empty_batch():
    q = torch.empty(0, 8, 128, dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros(2, 16, 2, 128, dtype=torch.bfloat16, device="cuda")
    idx = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    ak.ak_run_noalloc([0], [0], idx, [], 8, 2, 128, 16, q, kc, kc, out)
    # through ctypes directly: a null plan-options pointer is accepted
    dq, dk, do = ak.tensor_desc(q), ak.tensor_desc(kc), ak.tensor_desc(out)
    z = (ctypes.c_int32 * 1)(0)
    st = ak.lib().ak_run_noalloc(z, z, None, None, 0, 8, 2, 128, 16, 1, -1, None,
                                 ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dk),
                                 ctypes.byref(do), None, None)
    assert st == ak.AK_OK
