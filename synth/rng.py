"""Counter-based value generator shared by the oracle side and the device side.

Every value in a synthetic workload is a pure function of (seed, stream, index),
so any subset of a multi-gigabyte KV pool can be regenerated on the host (NumPy)
or on the device (torch integer ops on the GPU) and the two agree bit for bit.

The integer mixer is Thomas Mueller's 32-bit hash
    x = ((x >> 16) ^ x) * 0x45d9f3b;  x = ((x >> 16) ^ x) * 0x45d9f3b;  x = (x >> 16) ^ x
taken modulo 2^32.  The multiplier has 27 bits, so every product of a 32-bit
value fits in a signed 64-bit integer and the same arithmetic is exact in NumPy
int64 and torch int64 on any device.

Sixteen bits of the mixed counter select one entry of a 65,536-entry table of
standard-normal quantiles, ndtri((u + 0.5) / 65536).  The float32 table feeds
fp32 workloads; the bf16 table is the float32 table with its low 16 bits cleared
(truncation), so every generated bf16 value is exactly representable and no
rounding of the method under test is involved in producing inputs.

This module holds no arithmetic of the attention method: it only draws inputs.
"""

from __future__ import annotations

import numpy as np
from scipy.special import ndtri

MASK32 = 0xFFFFFFFF
MUL = 0x45D9F3B

# Named sub-streams; the value is mixed into the key so that streams never collide.
STREAMS = {"q": 1, "k_pool": 2, "v_pool": 3, "k_new": 4, "v_new": 5}


def _mix_py(x: int) -> int:
    x &= MASK32
    x = (((x >> 16) ^ x) * MUL) & MASK32
    x = (((x >> 16) ^ x) * MUL) & MASK32
    return ((x >> 16) ^ x) & MASK32


def stream_keys(seed: int, stream: str) -> tuple[int, int]:
    """Two 32-bit keys for (seed, stream); computed with Python integers."""
    sid = STREAMS[stream]
    k1 = _mix_py(_mix_py(seed * 2654435761 + sid) ^ 0x5BD1E995)
    k2 = _mix_py(k1 ^ 0x27D4EB2F)
    return k1, k2


def _normal_table_f32() -> np.ndarray:
    u = (np.arange(65536, dtype=np.float64) + 0.5) / 65536.0
    return ndtri(u).astype(np.float32)


TABLE_F32 = _normal_table_f32()
# bf16 table: float32 bit patterns truncated to their top 16 bits.
TABLE_BF16_BITS = (TABLE_F32.view(np.uint32) >> 16).astype(np.uint16)
TABLE_BF16_AS_F32 = (TABLE_BF16_BITS.astype(np.uint32) << 16).view(np.float32)


def max_abs(dtype: str) -> float:
    """Largest magnitude the generator can emit for a dtype ('f32' or 'bf16')."""
    t = TABLE_F32 if dtype == "f32" else TABLE_BF16_AS_F32
    return float(np.max(np.abs(t)))


# ---------------------------------------------------------------- host (NumPy)

def _mix_np(x: np.ndarray) -> np.ndarray:
    x = x & MASK32
    x = (((x >> 16) ^ x) * MUL) & MASK32
    x = (((x >> 16) ^ x) * MUL) & MASK32
    return ((x >> 16) ^ x) & MASK32


def _mix_np_inplace(x: np.ndarray) -> np.ndarray:
    """_mix_np on an int64 array, in place (same values, fewer temporaries)."""
    x &= MASK32
    t = x >> 16
    x ^= t
    x *= MUL
    x &= MASK32
    t = x >> 16
    x ^= t
    x *= MUL
    x &= MASK32
    t = x >> 16
    x ^= t
    return x


def table_index_np(seed: int, stream: str, idx: np.ndarray, chunk: int = 1 << 20) -> np.ndarray:
    """16-bit table indices for counters `idx` (any integer array, < 2^40)."""
    k1, k2 = stream_keys(seed, stream)
    idx = np.asarray(idx, dtype=np.int64)
    shape = idx.shape
    flat = idx.reshape(-1)
    out = np.empty(flat.shape, dtype=np.int64)
    for s in range(0, len(flat), chunk):
        c = flat[s:s + chunk]
        hi = c >> 32
        h = c & MASK32
        h ^= k1
        _mix_np_inplace(h)
        hi ^= k2
        _mix_np_inplace(hi)
        h ^= hi
        _mix_np_inplace(h)
        h &= 0xFFFF
        out[s:s + chunk] = h
    return out.reshape(shape)


def values_np(seed: int, stream: str, idx: np.ndarray, dtype: str) -> np.ndarray:
    """Generated values at counters `idx` as float32 ('f32' or 'bf16' grid)."""
    t = table_index_np(seed, stream, idx)
    table = TABLE_F32 if dtype == "f32" else TABLE_BF16_AS_F32
    return table[t]


def bf16_bits_np(seed: int, stream: str, idx: np.ndarray) -> np.ndarray:
    return TABLE_BF16_BITS[table_index_np(seed, stream, idx)]


# ------------------------------------------------------------- device (torch)

def _mix_t(x):
    x = x & MASK32
    x = (((x >> 16) ^ x) * MUL) & MASK32
    x = (((x >> 16) ^ x) * MUL) & MASK32
    return ((x >> 16) ^ x) & MASK32


_TORCH_TABLES: dict = {}


def _torch_table(device, dtype: str):
    import torch

    key = (str(device), dtype)
    if key not in _TORCH_TABLES:
        if dtype == "f32":
            t = torch.from_numpy(TABLE_F32.copy()).to(device)
        else:
            t = torch.from_numpy(TABLE_BF16_BITS.view(np.int16).copy()).to(device).view(torch.bfloat16)
        _TORCH_TABLES[key] = t
    return _TORCH_TABLES[key]


def fill_torch(out, seed: int, stream: str, start: int = 0, chunk: int = 1 << 27) -> None:
    """Fill a contiguous torch tensor with values at counters start .. start+numel.

    out.dtype must be torch.float32 (f32 grid) or torch.bfloat16 (bf16 grid).
    Works on any device.  Each chunk is 45 elementwise launches on a GPU; chunks
    bound the int64 temporaries (a few GB at the default 2^27 elements) and keep
    the launch count low (a multi-GB pool takes tens of chunks, not hundreds).
    """
    import torch

    dtype = "f32" if out.dtype == torch.float32 else "bf16"
    assert out.dtype in (torch.float32, torch.bfloat16) and out.is_contiguous()
    flat = out.view(-1)
    table = _torch_table(out.device, dtype)
    k1, k2 = stream_keys(seed, stream)
    n = flat.numel()
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        idx = torch.arange(start + s, start + e, device=out.device, dtype=torch.int64)
        lo = idx & MASK32
        hi = idx >> 32
        h = _mix_t(lo ^ k1)
        h = _mix_t(h ^ _mix_t(hi ^ k2))
        flat[s:e] = table[h & 0xFFFF]
        del idx, lo, hi, h
