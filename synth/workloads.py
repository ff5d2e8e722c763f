"""Seeded synthetic workloads shaped like the pages' batches.

A workload fixes, for one batch:
  * per-request query lengths n_r and KV lengths L_r (L_r counts this step's
    new tokens, which the step stores before it attends),
  * the page pool geometry and a random page assignment,
  * the CSR page table handed to the planner (kv_indptr / kv_indices /
    last_page_len) and qo_indptr,
  * slot_mapping for the step's new tokens (position p of request r lands in
    page_r[p // B] * B + p % B),
  * head geometry, dtypes, causal flag and sliding windows.

The CSR arrays and slot_mapping are the caller's inputs to the method (a serving
engine builds them from its block table); they are built here with plain loops.
The oracle re-derives lengths and slots from them on its own and the CPU tests
cross-check the two.

Small integer draws (lengths, permutations) use NumPy's PCG64 seeded by
SeedSequence(seed).spawn(4) in the fixed order: lengths, page permutation,
spare slots, shuffle.  Tensor values (Q, the KV pool, new K/V) come from the
counter-based generator in synth.rng, so any subset can be regenerated anywhere.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

from . import rng


@dataclasses.dataclass
class Workload:
    name: str
    seed: int
    q_lens: np.ndarray          # int64 [R]  n_r
    kv_lens: np.ndarray         # int64 [R]  L_r (after this step's store)
    page_size: int
    num_pages: int              # pool pages P
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int
    q_dtype: str                # 'f32' | 'bf16'  (also the dtype of new K/V and of out)
    kv_dtype: str               # 'f32' | 'bf16' | 'fp8'
    causal: bool
    windows: tuple              # window_left values, -1 = none; one plan per entry
    req_pages: list             # list of int64 arrays: physical pages of request r
    # CSR inputs (int32, host)
    qo_indptr: np.ndarray
    kv_indptr: np.ndarray
    kv_indices: np.ndarray
    last_page_len: np.ndarray
    # store_kv inputs
    slot_mapping: np.ndarray    # int64 [N_new]
    new_token_rows: np.ndarray  # int64 [N_new]: which q row (token) each new K/V belongs to
    kv_scale: float = 1.0       # per-tensor fp8 scale for both K and V (1.0 otherwise)
    extra: dict = dataclasses.field(default_factory=dict)

    @property
    def batch_size(self) -> int:
        return len(self.q_lens)

    @property
    def group(self) -> int:
        return self.num_qo_heads // self.num_kv_heads

    @property
    def total_q(self) -> int:
        return int(self.q_lens.sum())

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def pool_slots(self) -> int:
        return self.num_pages * self.page_size

    @property
    def pool_dtype(self) -> str:
        """dtype of the generated pool values before any quantisation."""
        return "f32" if self.kv_dtype == "f32" else "bf16"


def _csr(req_pages, kv_lens, q_lens, page_size):
    R = len(req_pages)
    kv_indptr = np.zeros(R + 1, dtype=np.int32)
    qo_indptr = np.zeros(R + 1, dtype=np.int32)
    last = np.zeros(R, dtype=np.int32)
    flat = []
    for r in range(R):
        kv_indptr[r + 1] = kv_indptr[r] + len(req_pages[r])
        qo_indptr[r + 1] = qo_indptr[r] + int(q_lens[r])
        used_in_last = int(kv_lens[r]) - (len(req_pages[r]) - 1) * page_size
        last[r] = used_in_last if len(req_pages[r]) else 0
        flat.extend(int(p) for p in req_pages[r])
    return qo_indptr, kv_indptr, np.asarray(flat, dtype=np.int32), last


def _new_token_slots(req_pages, kv_lens, q_lens, page_size):
    slots, rows = [], []
    row = 0
    for r in range(len(req_pages)):
        n, L = int(q_lens[r]), int(kv_lens[r])
        for j in range(n):
            p = L - n + j
            if p >= 0:   # a query before the cached positions (non-causal, n > L) stores nothing
                slots.append(int(req_pages[r][p // page_size]) * page_size + p % page_size)
                rows.append(row)
            row += 1
    return np.asarray(slots, dtype=np.int64), np.asarray(rows, dtype=np.int64)


def _assemble(name, seed, q_lens, kv_lens, page_size, perm_rng, hq, hkv, d, q_dtype,
              kv_dtype, causal, windows, spare_pages=0, token_granular=False, extra=None):
    q_lens = np.asarray(q_lens, dtype=np.int64)
    kv_lens = np.asarray(kv_lens, dtype=np.int64)
    pages_needed = [int(-(-int(L) // page_size)) for L in kv_lens]
    num_pages = sum(pages_needed) + spare_pages
    perm = perm_rng.permutation(num_pages).astype(np.int64)
    req_pages, off = [], 0
    for c in pages_needed:
        req_pages.append(perm[off:off + c])
        off += c
    qo_indptr, kv_indptr, kv_indices, last = _csr(req_pages, kv_lens, q_lens, page_size)
    slots, rows = _new_token_slots(req_pages, kv_lens, q_lens, page_size)
    scale = 1.0
    if kv_dtype == "fp8":
        # per-tensor scale: the largest magnitude the bf16 generator emits, over 448
        scale = float(np.float32(rng.max_abs("bf16")) / np.float32(448.0))
    return Workload(name=name, seed=seed, q_lens=q_lens, kv_lens=kv_lens, page_size=page_size,
                    num_pages=num_pages, num_qo_heads=hq, num_kv_heads=hkv, head_dim=d,
                    q_dtype=q_dtype, kv_dtype=kv_dtype, causal=causal, windows=tuple(windows),
                    req_pages=req_pages, qo_indptr=qo_indptr, kv_indptr=kv_indptr,
                    kv_indices=kv_indices, last_page_len=last, slot_mapping=slots,
                    new_token_rows=rows, kv_scale=scale, extra=extra or {})


def _streams(seed):
    ss = np.random.SeedSequence(seed).spawn(4)
    return [np.random.Generator(np.random.PCG64(s)) for s in ss]


# ------------------------------------------------------------------ the five

def tiny_decode(seed: int = 1) -> Workload:
    """4 decode requests, L = {7,16,33,64}, B = 16, pages from a permutation of a
    32-page pool, 4 q / 2 kv heads, D = 64, fp32, scale 1/8.  Each request's
    newest token is stored to its own slot (reading A); `extra['free_slots']`
    holds 4 distinct slots drawn from the 23 unallocated pages (reading B)."""
    g_len, g_perm, g_spare, _ = _streams(seed)
    kv_lens = [7, 16, 33, 64]
    wl = _assemble("tiny_decode_fp32", seed, [1, 1, 1, 1], kv_lens, 16, g_perm, 4, 2, 64,
                   "f32", "f32", True, (-1,), spare_pages=32 - 9)
    used = set(int(p) for p in wl.kv_indices)
    free_pages = [p for p in range(wl.num_pages) if p not in used]
    free_slots = np.asarray([p * 16 + o for p in free_pages for o in range(16)], dtype=np.int64)
    wl.extra["free_slots"] = g_spare.choice(free_slots, size=4, replace=False).astype(np.int64)
    return wl


def llama8b_decode(seed: int = 2, R: int = 64) -> Workload:
    """64 decode requests, L ~ U{512..8192}, B = 16, 32 q / 8 kv heads, D = 128,
    bf16, pages a random permutation of the pool (64 spare pages)."""
    g_len, g_perm, _, _ = _streams(seed)
    kv_lens = g_len.integers(512, 8192, size=R, endpoint=True)
    return _assemble("llama8b_decode_bf16", seed, np.ones(R, dtype=np.int64), kv_lens, 16,
                     g_perm, 32, 8, 128, "bf16", "bf16", True, (-1,), spare_pages=64)


def small_batch_decode(seed: int = 7, R: int = 8, lo: int = 256, hi: int = 1024) -> Workload:
    """A few short decode requests (the launch-bound regime graph replay is for):
    L ~ U{lo..hi}, otherwise shaped like llama8b_decode."""
    g_len, g_perm, _, _ = _streams(seed)
    kv_lens = g_len.integers(lo, hi, size=R, endpoint=True)
    return _assemble("small_batch_decode_bf16", seed, np.ones(R, dtype=np.int64), kv_lens, 16,
                     g_perm, 32, 8, 128, "bf16", "bf16", True, (-1,), spare_pages=16)


def ragged_prefill(seed: int = 3, R: int = 8, n_range=(128, 2048), p_range=(0, 4096)) -> Workload:
    """8 extend requests, n ~ U{128..2048} new tokens over a cached prefix
    p ~ U{0..4096}, causal aligned to the sequence end, B = 1 (indices are token
    slots, last_page_len = 1), slots a random permutation, 32/8 heads, D = 128, bf16."""
    g_len, g_perm, _, _ = _streams(seed)
    n = g_len.integers(n_range[0], n_range[1], size=R, endpoint=True)
    p = g_len.integers(p_range[0], p_range[1], size=R, endpoint=True)
    return _assemble("ragged_prefill_bf16", seed, n, n + p, 1, g_perm, 32, 8, 128, "bf16",
                     "bf16", True, (-1,), extra={"prefix": p})


def mixed_chunk_decode(seed: int = 4, R_dec: int = 255, chunk: int = 2048, prefix: int = 6144,
                       lmin: int = 1024, lmax: int = 32768, shuffle: bool = False) -> Workload:
    """One 2048-token prefill chunk over a 6144-token prefix plus 255 decode
    requests with L = round(exp(U[ln 1k, ln 32k])), B = 64, 32/8 heads, D = 128,
    bf16; two plans: full attention and sliding window 4096.  `shuffle` permutes
    the request order (the chunk is request 0 otherwise)."""
    g_len, g_perm, _, g_shuf = _streams(seed)
    dec = np.rint(np.exp(g_len.uniform(math.log(lmin), math.log(lmax), size=R_dec))).astype(np.int64)
    q_lens = np.concatenate([[chunk], np.ones(R_dec, dtype=np.int64)])
    kv_lens = np.concatenate([[chunk + prefix], dec])
    if shuffle:
        order = g_shuf.permutation(len(q_lens))
        q_lens, kv_lens = q_lens[order], kv_lens[order]
    return _assemble("mixed_chunk_decode_bf16", seed, q_lens, kv_lens, 64, g_perm, 32, 8, 128,
                     "bf16", "bf16", True, (-1, 4096))


def llama70b_long_decode(seed: int = 5, R: int = 8, L: int = 131072) -> Workload:
    """8 decode requests at 131072 tokens, 64 q / 8 kv heads, D = 128, bf16 Q,
    fp8 e4m3 K/V with one per-tensor fp32 scale, B = 64, permuted pages."""
    _, g_perm, _, _ = _streams(seed)
    return _assemble("llama70b_long_decode_fp8", seed, np.ones(R, dtype=np.int64),
                     np.full(R, L, dtype=np.int64), 64, g_perm, 64, 8, 128, "bf16", "fp8",
                     True, (-1,))


def shared_prefix_decode(seed: int = 6, R: int = 64, prefix_pages: int = 256,
                         suffix=(256, 2048)) -> Workload:
    """64 decode requests sharing their first 4096 tokens (256 pages of 16: one
    system prompt) followed by unique suffixes of U{256..2048} tokens; 32/8 heads,
    D = 128, bf16.  Every request's page list starts with the same pages;
    `extra['shared_pages']` is their count (the cascade's shared segment)."""
    g_len, g_perm, _, _ = _streams(seed)
    B = 16
    kv_lens = prefix_pages * B + g_len.integers(suffix[0], suffix[1], size=R, endpoint=True)
    wl = _assemble("shared_prefix_decode_bf16", seed, np.ones(R, dtype=np.int64), kv_lens, B,
                   g_perm, 32, 8, 128, "bf16", "bf16", True, (-1,))
    # request r's first prefix_pages pages become request 0's (its own first pages
    # stay allocated in the pool, unused); the new token sits in an unshared page
    for r in range(1, R):
        wl.req_pages[r][:prefix_pages] = wl.req_pages[0][:prefix_pages]
        a = int(wl.kv_indptr[r])
        wl.kv_indices[a:a + prefix_pages] = wl.kv_indices[:prefix_pages]
    wl.extra["shared_pages"] = prefix_pages
    return wl


CONFIGS = {
    1: tiny_decode,
    2: llama8b_decode,
    3: ragged_prefill,
    4: mixed_chunk_decode,
    5: llama70b_long_decode,
}


def config(k: int, **kw) -> Workload:
    return CONFIGS[k](seed=k, **kw)


# -------------------------------------------------------------- value access

def _elem_count_per_slot(wl: Workload) -> int:
    return wl.num_kv_heads * wl.head_dim


def pool_values(wl: Workload, which: str, slots: np.ndarray) -> np.ndarray:
    """Generated (pre-store, pre-quantisation) pool values at flat slots:
    float32 [len(slots), Hkv, D] on the f32 or bf16 grid."""
    per = _elem_count_per_slot(wl)
    slots = np.asarray(slots, dtype=np.int64)
    idx = slots[:, None] * per + np.arange(per, dtype=np.int64)[None, :]
    v = rng.values_np(wl.seed, f"{which}_pool", idx, wl.pool_dtype)
    return v.reshape(len(slots), wl.num_kv_heads, wl.head_dim)


def q_values(wl: Workload, rows: np.ndarray | None = None) -> np.ndarray:
    """Q values float32 [len(rows), Hq, D] (rows = global query-token indices)."""
    if rows is None:
        rows = np.arange(wl.total_q, dtype=np.int64)
    per = wl.num_qo_heads * wl.head_dim
    idx = np.asarray(rows, dtype=np.int64)[:, None] * per + np.arange(per, dtype=np.int64)[None, :]
    return rng.values_np(wl.seed, "q", idx, wl.q_dtype).reshape(len(rows), wl.num_qo_heads, wl.head_dim)


def new_kv_values(wl: Workload, which: str, rows: np.ndarray | None = None) -> np.ndarray:
    """This step's new K or V values float32 [len(rows), Hkv, D] on the q-dtype grid."""
    if rows is None:
        rows = np.arange(len(wl.slot_mapping), dtype=np.int64)
    per = _elem_count_per_slot(wl)
    idx = np.asarray(rows, dtype=np.int64)[:, None] * per + np.arange(per, dtype=np.int64)[None, :]
    return rng.values_np(wl.seed, f"{which}_new", idx, wl.q_dtype).reshape(
        len(rows), wl.num_kv_heads, wl.head_dim)


# ----------------------------------------------------------- device tensors

def torch_dtype(name: str):
    import torch

    return {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}[name]


def device_inputs(wl: Workload, device, with_pool: bool = True) -> dict:
    """Allocate and fill the workload's tensors on `device`.

    Returns q [ΣN, Hq, D], k_new / v_new [N_new, Hkv, D] (q dtype), slot_mapping
    int64, kv_indices int32 and, if `with_pool`, the pools:
      * f32 / bf16 caches: k_cache / v_cache [P, B, Hkv, D] already holding the
        generated pool values;
      * fp8 caches: uint8 k_cache / v_cache [P, B, Hkv, D] left uninitialised plus
        k_pool_src / v_pool_src (bf16, same shape) holding the values that the
        caller quantises into the cache with its own store.
    """
    import torch

    qd = torch_dtype(wl.q_dtype)
    out = {}
    out["q"] = torch.empty(wl.total_q, wl.num_qo_heads, wl.head_dim, dtype=qd, device=device)
    rng.fill_torch(out["q"], wl.seed, "q")
    nn = len(wl.slot_mapping)
    for w in ("k", "v"):
        t = torch.empty(nn, wl.num_kv_heads, wl.head_dim, dtype=qd, device=device)
        rng.fill_torch(t, wl.seed, f"{w}_new")
        out[f"{w}_new"] = t
    out["slot_mapping"] = torch.from_numpy(wl.slot_mapping.copy()).to(device)
    out["kv_indices"] = torch.from_numpy(wl.kv_indices.astype(np.int32)).to(device)
    if with_pool:
        shape = (wl.num_pages, wl.page_size, wl.num_kv_heads, wl.head_dim)
        for w in ("k", "v"):
            if wl.kv_dtype == "fp8":
                src = torch.empty(shape, dtype=torch.bfloat16, device=device)
                rng.fill_torch(src, wl.seed, f"{w}_pool")
                out[f"{w}_pool_src"] = src
                out[f"{w}_cache"] = torch.empty(shape, dtype=torch.uint8, device=device)
            else:
                c = torch.empty(shape, dtype=torch_dtype(wl.kv_dtype), device=device)
                rng.fill_torch(c, wl.seed, f"{w}_pool")
                out[f"{w}_cache"] = c
    return out


def custom(seed: int, q_lens, kv_lens, page_size: int, num_qo_heads: int, num_kv_heads: int,
           head_dim: int, q_dtype: str = "bf16", kv_dtype: str = "bf16", causal: bool = True,
           windows=(-1,), spare_pages: int = 3, name: str = "custom") -> Workload:
    """A workload with given per-request query and KV lengths (edge-case tests)."""
    _, g_perm, _, _ = _streams(seed)
    return _assemble(name, seed, q_lens, kv_lens, page_size, g_perm, num_qo_heads, num_kv_heads,
                     head_dim, q_dtype, kv_dtype, causal, windows, spare_pages=spare_pages)
