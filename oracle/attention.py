"""Paged-KV attention, the plain way: one request at a time, in float64.

Citations name the page and the section on it:
  [vLLM backend]  "vLLM attention backend" page: "Write the KV first"
                  (store-then-attend), the nine invariants (non-padding slots).
  [SGLang]        "SGLang attention backend" page: "Where masks come from"
                  (causal bit; sliding window keeps k >= q - w) and "The two
                  forms of extend" (merging two attention states by their
                  log-sum-exp).
  [mini-sglang]   "GPU attention" page of the mini-sglang handbook: the CPU
                  reference paged attention of the "Verify on the CPU" section
                  (gather K/V through the page list, queries are the last n
                  positions, causal mask aligned bottom-right, GQA, default
                  scale 1/sqrt(D)).

Readings where the pages leave a step open:
  * GQA map: query head h reads KV head h // (Hq / Hkv) (consecutive groups).
  * Window: window_left = w >= 0 keeps keys t with q_pos - w <= t (w + 1 keys
    with the causal bound); w = -1 means no window.
  * LSE: natural logarithm of the sum of exp(scaled logits).
  * Merge operands: each part's output normalised by its own sum, with its LSE.
  * slot_mapping: int64; a negative slot marks padding and is skipped.
"""

from __future__ import annotations

import math

import numpy as np

from . import codecs
from .metadata import kv_lengths, q_lengths, request_slots

# -------------------------------------------------------------------- cache

class Cache:
    """A K or V pool held as stored codes: float32 values, bf16 bit patterns
    (uint16) or E4M3 codes (uint8) with a per-tensor scale.
    Shape [num_pages, page_size, num_kv_heads, head_dim]."""

    def __init__(self, codes: np.ndarray, dtype: str, scale: float = 1.0):
        self.codes = codes
        self.dtype = dtype
        self.scale = float(scale)

    @property
    def page_size(self):
        return self.codes.shape[1]

    def flat(self):
        c = self.codes
        return c.reshape(c.shape[0] * c.shape[1], c.shape[2], c.shape[3])

    def decode_slots(self, slots) -> np.ndarray:
        """Stored values at flat slots as float64 [len(slots), Hkv, D]."""
        c = self.flat()[np.asarray(slots, dtype=np.int64)]
        if self.dtype == "f32":
            return c.astype(np.float64)
        if self.dtype == "bf16":
            return codecs.bf16_decode(c)
        return codecs.e4m3_decode(c, self.scale)


def encode(values_f32: np.ndarray, dtype: str, scale: float = 1.0) -> np.ndarray:
    """Encode binary32 values into the cache's stored form."""
    v = np.asarray(values_f32, dtype=np.float32)
    if dtype == "f32":
        return v.copy()
    if dtype == "bf16":
        return codecs.bf16_encode(v)
    return codecs.e4m3_encode(v, scale)


def store_kv(cache: Cache, new_values_f32: np.ndarray, slot_mapping) -> None:
    """Write token i's [Hkv, D] values into flat slot slot_mapping[i], in order.

    Negative slots are padding and are skipped.  The write happens before any
    attention over the cache in the same step.  [vLLM backend, write-first]
    """
    flat = cache.flat()
    enc = encode(new_values_f32, cache.dtype, cache.scale)
    for i, s in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if s >= 0:
            flat[s] = enc[i]


# ---------------------------------------------------------------- attention

def attend_one(q, K, V, q_pos, sm_scale, causal, window, kv_range=None):
    """Attention of one query head's rows over one KV head's keys.

    q [n, D], K/V [L, D] float64, q_pos [n] absolute positions of the queries.
    Returns out [n, D] and lse [n] (natural log).  `kv_range = (a, b)` limits
    the keys to positions a .. b-1 (used to form split-KV parts); a row with no
    visible key in the range gets out = 0 and lse = -inf.
    """
    n, D = q.shape
    L = K.shape[0]
    t = np.arange(L)[None, :]
    qp = np.asarray(q_pos)[:, None]
    visible = np.ones((n, L), dtype=bool)
    if causal:
        visible &= t <= qp
    if window is not None and window >= 0:
        visible &= t >= qp - window
    if kv_range is not None:
        visible &= (t >= kv_range[0]) & (t < kv_range[1])
    s = sm_scale * (q @ K.T)                       # [n, L]
    s = np.where(visible, s, -np.inf)
    m = np.max(s, axis=1, keepdims=True)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    p = np.where(visible, np.exp(s - m_safe), 0.0)
    ell = p.sum(axis=1, keepdims=True)
    with np.errstate(invalid="ignore", divide="ignore"):
        out = np.where(ell > 0, (p @ V) / np.where(ell > 0, ell, 1.0), 0.0)
        lse = np.where(ell[:, 0] > 0, m_safe[:, 0] + np.log(np.where(ell[:, 0] > 0, ell[:, 0], 1.0)),
                       -np.inf)
    return out, lse


def paged_attention(q, k_cache: Cache, v_cache: Cache, qo_indptr, kv_indptr, kv_indices,
                    last_page_len, num_kv_heads, sm_scale=None, causal=True, window=-1,
                    requests=None, kv_range_of=None, rows_of=None):
    """Batched paged attention, request by request.

    q: float64 [sum n, Hq, D].  For request r: gather K/V of positions 0..L_r-1
    through its page list, place its n_r queries at positions L_r - n_r + j,
    and attend with query head h reading KV head h // G.
    `requests` limits the work to some requests (others are left as NaN).
    `kv_range_of(r)` optionally gives a key range per request (split parts).
    `rows_of(r)` optionally lists which of request r's query indices j to compute
    (each query row is computed independently of the others).
    Returns out float64 [sum n, Hq, D], lse float64 [sum n, Hq].
    """
    q = np.asarray(q, dtype=np.float64)
    T, Hq, D = q.shape
    B = k_cache.page_size
    G = Hq // num_kv_heads
    scale = (1.0 / math.sqrt(D)) if sm_scale is None else float(sm_scale)
    Ls = kv_lengths(kv_indptr, last_page_len, B)
    ns = q_lengths(qo_indptr)
    out = np.full((T, Hq, D), np.nan)
    lse = np.full((T, Hq), np.nan)
    todo = range(len(ns)) if requests is None else requests
    for r in todo:
        n, L = int(ns[r]), int(Ls[r])
        if n == 0:
            continue
        q0 = int(qo_indptr[r])
        slots = request_slots(kv_indptr, kv_indices, last_page_len, B, r)
        K = k_cache.decode_slots(slots)                     # [L, Hkv, D]
        V = v_cache.decode_slots(slots)
        js = np.arange(n) if rows_of is None else np.asarray(rows_of(r), dtype=np.int64)
        q_pos = L - n + js
        rng_r = None if kv_range_of is None else kv_range_of(r)
        for h in range(Hq):
            hk = h // G
            o, l = attend_one(q[q0 + js, h, :], K[:, hk, :], V[:, hk, :], q_pos, scale,
                              causal, window, rng_r)
            out[q0 + js, h, :] = o
            lse[q0 + js, h] = l
    return out, lse


# -------------------------------------------------------------------- merge

def merge_states(outs, lses):
    """Merge attention states computed over disjoint key sets.

    m = max_s lse_s,  w_s = exp(lse_s - m),
    out = sum_s w_s out_s / sum_s w_s,  lse = m + ln(sum_s w_s).
    A part with lse = -inf has weight 0.  [SGLang, two forms of extend]
    outs: list of [..., D]; lses: list of [...].
    """
    L = np.stack([np.asarray(x, dtype=np.float64) for x in lses])          # [S, ...]
    O = np.stack([np.asarray(x, dtype=np.float64) for x in outs])          # [S, ..., D]
    m = np.max(L, axis=0)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    w = np.where(np.isfinite(L), np.exp(L - m_safe), 0.0)
    wsum = w.sum(axis=0)
    with np.errstate(invalid="ignore", divide="ignore"):
        out = (w[..., None] * O).sum(axis=0) / np.where(wsum > 0, wsum, 1.0)[..., None]
        lse = np.where(wsum > 0, m_safe + np.log(np.where(wsum > 0, wsum, 1.0)), -np.inf)
    return out, lse
