"""Run the oracle on a synthetic workload (test infrastructure only).

The KV pools of the large workloads are gigabytes, so the oracle never builds
them whole: `GeneratedCache` produces the stored code of any slot on demand --
the generated pool value encoded with the oracle's own codec, unless this
step's store overwrote the slot.
"""

from __future__ import annotations

import numpy as np

from synth import workloads as W

from . import attention as A


class GeneratedCache:
    # slots generated per piece; large requests are generated piece by piece on a
    # few host threads (NumPy releases the interpreter lock inside its array
    # operations), which changes nothing in the codes, only the wall time
    piece_slots = 8192
    threads = 8

    def __init__(self, wl: W.Workload, which: str):
        self.wl = wl
        self.which = which
        self.dtype = wl.kv_dtype
        self.scale = wl.kv_scale
        self.page_size = wl.page_size
        self.overlay: dict = {}

    def store(self, new_values_f32: np.ndarray, slot_mapping) -> None:
        """Same write rule as attention.store_kv, into the overlay."""
        enc = A.encode(new_values_f32, self.dtype, self.scale)
        for i, s in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
            if s >= 0:
                self.overlay[int(s)] = enc[i]

    def materialize(self, slots) -> None:
        """Generate and keep the codes of these slots, so later reads of them do
        no input generation (used to time the oracle's own work only)."""
        slots = np.unique(np.asarray(slots, dtype=np.int64))
        self._pre_slots = None
        codes = self.codes_at(slots)
        self._pre_slots, self._pre_codes = slots, codes

    def _generated(self, slots: np.ndarray) -> np.ndarray:
        """Pool codes at these slots as generated (before this step's store)."""
        n, k = len(slots), self.piece_slots
        if n <= k:
            return A.encode(W.pool_values(self.wl, self.which, slots), self.dtype, self.scale)
        import concurrent.futures

        pieces = [slots[i:i + k] for i in range(0, n, k)]
        with concurrent.futures.ThreadPoolExecutor(self.threads) as ex:
            parts = list(ex.map(lambda sl: A.encode(W.pool_values(self.wl, self.which, sl),
                                                    self.dtype, self.scale), pieces))
        return np.concatenate(parts)

    def codes_at(self, slots) -> np.ndarray:
        slots = np.asarray(slots, dtype=np.int64)
        pre = getattr(self, "_pre_slots", None)
        if pre is not None:
            pos = np.searchsorted(pre, slots)
            pos = np.clip(pos, 0, len(pre) - 1)
            if np.all(pre[pos] == slots):
                return self._pre_codes[pos]
        base = self._generated(slots)
        if self.overlay:
            keys = np.fromiter(self.overlay.keys(), dtype=np.int64, count=len(self.overlay))
            for i in np.nonzero(np.isin(slots, keys))[0]:
                base[i] = self.overlay[int(slots[i])]
        return base

    def decode_slots(self, slots) -> np.ndarray:
        c = self.codes_at(slots)
        tmp = A.Cache(c[:, None], self.dtype, self.scale)   # [n, 1, Hkv, D]
        return tmp.decode_slots(np.arange(len(c)))


def caches_after_store(wl: W.Workload, slot_mapping=None, new_rows=None):
    """K and V caches of the workload after this step's store_kv."""
    kc, vc = GeneratedCache(wl, "k"), GeneratedCache(wl, "v")
    sm = wl.slot_mapping if slot_mapping is None else slot_mapping
    rows = np.arange(len(sm)) if new_rows is None else new_rows
    kc.store(W.new_kv_values(wl, "k", rows), sm)
    vc.store(W.new_kv_values(wl, "v", rows), sm)
    return kc, vc


def decoded_q(wl: W.Workload) -> np.ndarray:
    return W.q_values(wl).astype(np.float64)


def run(wl: W.Workload, window: int = -1, requests=None, caches=None, q=None, rows_of=None):
    """Oracle out/lse (float64) for the workload, optionally for some requests
    (and some query rows of them) only; rows not computed are NaN."""
    kc, vc = caches if caches is not None else caches_after_store(wl)
    qq = decoded_q(wl) if q is None else q
    return A.paged_attention(qq, kc, vc, wl.qo_indptr, wl.kv_indptr, wl.kv_indices,
                             wl.last_page_len, wl.num_kv_heads, sm_scale=wl.sm_scale,
                             causal=wl.causal, window=window, requests=requests,
                             rows_of=rows_of)
