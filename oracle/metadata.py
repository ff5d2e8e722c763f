"""Batch metadata of a paged KV cache: CSR page table, lengths and slots.

Citations name the page and the section on it:
  [vLLM backend]  "vLLM attention backend" page -- sections "From a 2-D block
                  table to a CSR page table" and the worked example with
                  requests A/B/C.
  [mini-sglang]   "GPU attention" page of the mini-sglang handbook -- sections
                  "FlashInfer: plan and run", "FlashAttention: page-number
                  table" and the example run.

The display formulas of the CSR section were lost from the page text; the
readings below are restored from the page's prose and from the worked example's
printed numbers, which they reproduce exactly:
  pages_i       = ceil(l_i / B)
  kv_indptr     = [0, prefix sums of pages_i]
  last_page_len = l_i - (pages_i - 1) * B, which lies in [1, B] (a full last
                  page is B, never 0)
  slot(pos)     = block_row[pos // B] * B + pos % B
"""

from __future__ import annotations

import numpy as np


def block_table_to_csr(seq_lens, block_rows, page_size):
    """2-D block-table rows -> (kv_indptr, kv_indices, last_page_len).

    Only the first ceil(l_i / B) entries of row i are valid; the rest is padding.
    [vLLM backend, CSR section]
    """
    B = int(page_size)
    pages = [-(-int(l) // B) for l in seq_lens]
    indptr = [0]
    for p in pages:
        indptr.append(indptr[-1] + p)
    indices = []
    for row, p in zip(block_rows, pages):
        indices.extend(int(x) for x in list(row)[:p])
    last = [int(l) - (p - 1) * B if p > 0 else 0 for l, p in zip(seq_lens, pages)]
    return (np.asarray(indptr, dtype=np.int64), np.asarray(indices, dtype=np.int64),
            np.asarray(last, dtype=np.int64))


def virtual_block_rows(block_rows, ratio):
    """Manager-block rows -> kernel-page rows.

    A manager block of M = ratio * B tokens is exposed to a kernel that takes
    B-token pages as `ratio` virtual kernel blocks; the expansion has to agree
    with the cache view, so block b of a cache [P, M, Hkv, D] becomes pages
    b * ratio + i (i < ratio) of the same memory viewed as [P * ratio, B, Hkv, D].
    [vLLM backend, "Hybrid KV and virtual kernel blocks"; the formula is the
    reading that keeps every flat slot unchanged]
    """
    ratio = int(ratio)
    return [[int(b) * ratio + i for b in row for i in range(ratio)] for row in block_rows]


def kv_lengths(kv_indptr, last_page_len, page_size):
    """CSR page table -> KV length of every request.

    L_r = (pages_r - 1) * B + last_page_len[r]; a request with no pages has L_r = 0.
    """
    indptr = np.asarray(kv_indptr, dtype=np.int64)
    pages = indptr[1:] - indptr[:-1]
    last = np.asarray(last_page_len, dtype=np.int64)
    return np.where(pages > 0, (pages - 1) * int(page_size) + last, 0)


def q_lengths(qo_indptr):
    p = np.asarray(qo_indptr, dtype=np.int64)
    return p[1:] - p[:-1]


def slot_of(block_row, pos, page_size):
    """Flat cache slot of logical position `pos` of one request.
    [vLLM backend, worked example: position 127 of A -> page 7 offset 15 -> slot 175]"""
    B = int(page_size)
    return int(block_row[int(pos) // B]) * B + int(pos) % B


def slot_mapping(block_rows, positions_per_request, page_size):
    """Write slots of every new token, requests in batch order."""
    out = []
    for row, positions in zip(block_rows, positions_per_request):
        out.extend(slot_of(row, p, page_size) for p in positions)
    return np.asarray(out, dtype=np.int64)


def request_slots(kv_indptr, kv_indices, last_page_len, page_size, r):
    """Flat slots of positions 0 .. L_r-1 of request r, read through its page list."""
    indptr = np.asarray(kv_indptr, dtype=np.int64)
    pages = np.asarray(kv_indices, dtype=np.int64)[indptr[r]:indptr[r + 1]]
    L = int(kv_lengths(indptr[r:r + 2], np.asarray(last_page_len)[r:r + 1], page_size)[0])
    B = int(page_size)
    return np.asarray([int(pages[t // B]) * B + t % B for t in range(L)], dtype=np.int64)


def split_decode_prefill(qo_indptr, threshold=1):
    """Classify requests by query length and slice qo_indptr per phase.

    Requests with a query length at or below `threshold` are decodes.  Each
    phase's qo_indptr is the sub-array of its requests rebased to start at 0.
    [vLLM backend, worked example: [0,1,5,8] -> decode A, prefill slice [0,4,7]]
    """
    q = q_lengths(qo_indptr)
    dec = [i for i, n in enumerate(q) if n <= threshold]
    pre = [i for i, n in enumerate(q) if n > threshold]

    def sub(ids):
        p = [0]
        for i in ids:
            p.append(p[-1] + int(q[i]))
        return np.asarray(p, dtype=np.int64)

    return dec, sub(dec), pre, sub(pre)


def token_view(kv_indptr, kv_indices, last_page_len, page_size):
    """Rewrite a page-granular CSR as the page_size = 1 view of the same pool:
    indices become token slots and every last_page_len becomes 1.
    [mini-sglang, FlashInfer section: the pool is viewed as [tokens, 1, H, D]]"""
    indptr = np.asarray(kv_indptr, dtype=np.int64)
    R = len(indptr) - 1
    new_indptr = [0]
    flat = []
    for r in range(R):
        s = request_slots(indptr, kv_indices, last_page_len, page_size, r)
        flat.extend(int(x) for x in s)
        new_indptr.append(new_indptr[-1] + len(s))
    return (np.asarray(new_indptr, dtype=np.int64), np.asarray(flat, dtype=np.int64),
            np.ones(R, dtype=np.int64))


def page_table_from_token_table(token_rows, seq_lens, page_size):
    """Token-position table -> page-number table: keep every B-th entry of a row
    (the first slot of each page) and floor-divide it by B.
    [mini-sglang, FlashAttention section]"""
    B = int(page_size)
    out = []
    for row, L in zip(token_rows, seq_lens):
        n_pages = -(-int(L) // B)
        out.append([int(row[k * B]) // B for k in range(n_pages)])
    return out
