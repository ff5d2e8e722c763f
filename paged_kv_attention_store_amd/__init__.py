"""Python binding of libak -- batched paged-KV attention on AMD MI355X (gfx950).

A thin ctypes layer over the C ABI in include/ak.h: it marshals torch tensors
into `ak_tensor` descriptors (data pointer, dtype, shape, strides) and passes the
current HIP stream.  Every step of the computation runs in libak's kernels;
torch only provides device memory and streams.  If libak.so is missing or fails
to load, importing this package raises -- there is no other implementation.

Entry points (same names as the C ABI):
    ak_store_kv(k, v, slot_mapping, k_cache, v_cache, k_scale=1.0, v_scale=1.0)
    ak_plan(qo_indptr, kv_indptr, kv_indices, last_page_len, num_qo_heads,
            num_kv_heads, head_dim, page_size, causal=True, window=-1, ...) -> Plan
    ak_run(plan, q, k_cache, v_cache, out=None, lse=None, k_scale=1.0, v_scale=1.0)
    ak_merge_states(o_a, lse_a, o_b, lse_b, out=None, lse_out=None)
    ak_run_noalloc(qo_indptr, kv_indptr, kv_indices, last_page_len, ..., q, k_cache,
                   v_cache, out, lse)   (plan + run without allocating)
    ak_plan_destroy, ak_plan_info, ak_plan_export, ak_gather_slots,
    ak_profile_enable, ak_profile_read, ak_last_error, ak_version
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libak.so")

# status codes and dtypes, mirroring include/ak.h
AK_OK = 0
AK_ERR_INVALID_ARG = -1
AK_ERR_UNSUPPORTED = -2
AK_ERR_BAD_INDPTR = -3
AK_ERR_BAD_LENGTHS = -4
AK_ERR_SHAPE_MISMATCH = -5
AK_ERR_HIP = -6
AK_ERR_OOM = -7
STATUS_NAMES = {0: "AK_OK", -1: "AK_ERR_INVALID_ARG", -2: "AK_ERR_UNSUPPORTED",
                -3: "AK_ERR_BAD_INDPTR", -4: "AK_ERR_BAD_LENGTHS", -5: "AK_ERR_SHAPE_MISMATCH",
                -6: "AK_ERR_HIP", -7: "AK_ERR_OOM"}

AK_F32, AK_BF16, AK_FP8_E4M3, AK_I32, AK_I64 = 0, 1, 2, 3, 4
AK_PLAN_HOST_ONLY = 1
AK_PLAN_MERGE_IN_KERNEL = 2
AK_PLAN_SHARED_PAGES = 4
AK_PLAN_STREAM_K = 8
AK_PROFILE_ALL = 0x1F

EXPORTED = ["ak_store_kv", "ak_plan", "ak_plan_destroy", "ak_run", "ak_last_error",
            "ak_plan_info", "ak_plan_export", "ak_gather_slots", "ak_profile_enable",
            "ak_merge_states", "ak_csr_from_block_table", "ak_slot_mapping", "ak_plan_fixed",
            "ak_plan_update",
            "ak_profile_read", "ak_version", "ak_fp8_to_bf16", "ak_run_noalloc",
            "ak_plan_workgroups"]


class AkError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class AkTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("stride", ctypes.c_int64 * 4),
                ("scale", ctypes.c_float)]


class AkPlanOpts(ctypes.Structure):
    _fields_ = [("sm_scale", ctypes.c_float), ("num_cus", ctypes.c_int32),
                ("max_splits", ctypes.c_int32), ("min_chunk", ctypes.c_int32),
                ("flags", ctypes.c_int32), ("stream", ctypes.c_void_p)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libak.so not found at {LIB_PATH}; build it with "
                          "`python -c 'import __graft_entry__ as g; g.build()'`")
    # torch ships its own HIP runtime and loads it by path; libak must bind to
    # that same runtime (one runtime per process), so torch is loaded first
    try:
        import torch  # noqa: F401
    except ImportError:  # pragma: no cover - the host-only planner still works
        pass
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    i32p = P(ctypes.c_int32)
    lib.ak_store_kv.argtypes = [P(AkTensor)] * 5 + [ctypes.c_void_p]
    lib.ak_store_kv.restype = ctypes.c_int
    lib.ak_plan.argtypes = [i32p, i32p, ctypes.c_void_p, i32p] + [ctypes.c_int32] * 7 + [
        P(AkPlanOpts), P(ctypes.c_void_p)]
    lib.ak_plan.restype = ctypes.c_int
    lib.ak_plan_fixed.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                  ctypes.c_void_p] + [
        ctypes.c_int32] * 6 + [P(AkPlanOpts), P(ctypes.c_void_p)]
    lib.ak_plan_fixed.restype = ctypes.c_int
    lib.ak_plan_update.argtypes = [ctypes.c_void_p, i32p, i32p, i32p, ctypes.c_int32, ctypes.c_void_p]
    lib.ak_plan_update.restype = ctypes.c_int
    lib.ak_plan_destroy.argtypes = [ctypes.c_void_p]
    lib.ak_plan_destroy.restype = None
    lib.ak_run.argtypes = [ctypes.c_void_p] + [P(AkTensor)] * 5 + [ctypes.c_void_p]
    lib.ak_run.restype = ctypes.c_int
    lib.ak_run_noalloc.argtypes = [i32p, i32p, ctypes.c_void_p, i32p] + [ctypes.c_int32] * 7 + [
        P(AkPlanOpts)] + [P(AkTensor)] * 5 + [ctypes.c_void_p]
    lib.ak_run_noalloc.restype = ctypes.c_int
    lib.ak_last_error.argtypes = []
    lib.ak_last_error.restype = ctypes.c_char_p
    lib.ak_plan_info.argtypes = [ctypes.c_void_p, P(ctypes.c_int64), ctypes.c_int32]
    lib.ak_plan_info.restype = ctypes.c_int
    lib.ak_plan_export.argtypes = [ctypes.c_void_p, i32p, ctypes.c_int64, P(ctypes.c_int64), i32p]
    lib.ak_plan_export.restype = ctypes.c_int
    lib.ak_plan_workgroups.argtypes = [ctypes.c_void_p, i32p, ctypes.c_int64, P(ctypes.c_int64)]
    lib.ak_plan_workgroups.restype = ctypes.c_int
    lib.ak_merge_states.argtypes = [P(AkTensor)] * 6 + [ctypes.c_void_p]
    lib.ak_merge_states.restype = ctypes.c_int
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.ak_csr_from_block_table.argtypes = [vp, i64, vp, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_int32, vp, vp, i64, vp, vp]
    lib.ak_csr_from_block_table.restype = ctypes.c_int
    lib.ak_slot_mapping.argtypes = [vp, i64, vp, vp, ctypes.c_int32, ctypes.c_int32, vp, i64, vp]
    lib.ak_slot_mapping.restype = ctypes.c_int
    lib.ak_gather_slots.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    lib.ak_gather_slots.restype = ctypes.c_int
    lib.ak_profile_enable.argtypes = [ctypes.c_int32]
    lib.ak_profile_enable.restype = ctypes.c_int
    lib.ak_profile_read.argtypes = [P(ctypes.c_int64), P(ctypes.c_double), ctypes.c_int32]
    lib.ak_profile_read.restype = ctypes.c_int
    lib.ak_fp8_to_bf16.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.ak_fp8_to_bf16.restype = ctypes.c_int
    lib.ak_version.argtypes = []
    lib.ak_version.restype = ctypes.c_char_p
    return lib


_lib = _load()


def lib():
    return _lib


def ak_last_error() -> str:
    return _lib.ak_last_error().decode()


def ak_version() -> str:
    return _lib.ak_version().decode()


def _check(status: int):
    if status != AK_OK:
        raise AkError(status, ak_last_error())


# ------------------------------------------------------------ marshalling

def _dtype_code(t) -> int:
    import torch

    m = {torch.float32: AK_F32, torch.bfloat16: AK_BF16, torch.uint8: AK_FP8_E4M3,
         torch.float8_e4m3fn: AK_FP8_E4M3, torch.int32: AK_I32, torch.int64: AK_I64}
    if t.dtype not in m:
        raise TypeError(f"unsupported tensor dtype {t.dtype}")
    return m[t.dtype]


def tensor_desc(t, scale: float = 1.0) -> AkTensor:
    """Describe a torch tensor (device memory) for the C ABI."""
    if t.dim() > 4:
        raise ValueError("at most 4 dimensions")
    d = AkTensor()
    d.data = t.data_ptr() if t.numel() > 0 else None
    d.dtype = _dtype_code(t)
    d.ndim = t.dim()
    for i in range(t.dim()):
        d.shape[i] = t.shape[i]
        d.stride[i] = t.stride(i)
    d.scale = float(scale)
    return d


_DESC_CACHE: dict = {}
_DESC_CACHE_MAX = 4096


def _desc(t, scale: float = 1.0) -> AkTensor:
    """tensor_desc for the entry points: a descriptor is a pure function of the
    tensor's address, dtype, shape, strides and scale, so one built earlier for
    the same values is reused (serving loops pass the same tensors every step).
    Shared objects: never modify what this returns."""
    key = (t.data_ptr(), t.dtype, t.shape, t.stride(), scale)
    d = _DESC_CACHE.get(key)
    if d is None:
        if len(_DESC_CACHE) >= _DESC_CACHE_MAX:
            _DESC_CACHE.clear()
        d = _DESC_CACHE[key] = tensor_desc(t, scale)
    return d


def _stream_ptr(stream):
    import torch

    if stream is None:
        if not torch.cuda.is_available():
            return ctypes.c_void_p(None)      # host-only paths never launch
        return ctypes.c_void_p(torch._C._cuda_getCurrentRawStream(torch.cuda.current_device()))
    return ctypes.c_void_p(stream.cuda_stream)


def _host_i32(a):
    arr = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    return arr, arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


# ------------------------------------------------------------ entry points

def ak_store_kv(k, v, slot_mapping, k_cache, v_cache, k_scale: float = 1.0, v_scale: float = 1.0,
                stream=None) -> None:
    """Scatter k/v [N, Hkv, D] into the caches [P, B, Hkv, D] at slot_mapping (int64)."""
    dk, dv, ds = _desc(k), _desc(v), _desc(slot_mapping)
    dkc, dvc = _desc(k_cache, k_scale), _desc(v_cache, v_scale)
    _check(_lib.ak_store_kv(ctypes.byref(dk), ctypes.byref(dv), ctypes.byref(ds),
                            ctypes.byref(dkc), ctypes.byref(dvc), _stream_ptr(stream)))


class Plan:
    """Owns an ak_plan_t; destroyed with the object (or by ak_plan_destroy)."""

    def __init__(self, handle, num_qo_heads, num_kv_heads, head_dim, page_size, host_only, keep):
        self.handle = handle
        self.num_qo_heads = num_qo_heads
        self.num_kv_heads = num_kv_heads
        self.head_dim = head_dim
        self.page_size = page_size
        self.host_only = host_only
        self._keep = keep           # the borrowed kv_indices tensor stays alive with the plan

    def __del__(self):
        destroy = globals().get("ak_plan_destroy")
        if destroy is not None:         # None while the interpreter shuts down
            destroy(self)

    def info(self) -> dict:
        return ak_plan_info(self)


def ak_plan(qo_indptr, kv_indptr, kv_indices, last_page_len, num_qo_heads: int, num_kv_heads: int,
            head_dim: int, page_size: int, causal: bool = True, window: int = -1,
            sm_scale: float | None = None, num_cus: int = 0, max_splits: int = 0,
            min_chunk: int = 0, host_only: bool = False, merge_in_kernel: bool = False,
            shared_pages: bool = False, stream_k: bool = False, stream=None) -> Plan:
    """Build a plan.  qo_indptr, kv_indptr and last_page_len are host arrays
    (anything NumPy accepts); kv_indices is a device int32 tensor (or None for a
    host-only plan).  stream_k selects the stream-K decode partition."""
    qo, qo_p = _host_i32(qo_indptr)
    kv, kv_p = _host_i32(kv_indptr)
    last, last_p = _host_i32(last_page_len)
    R = len(qo) - 1
    if len(kv) != R + 1 or len(last) != R:
        raise ValueError("qo_indptr/kv_indptr need batch_size+1 entries, last_page_len batch_size")
    opts = AkPlanOpts()
    opts.sm_scale = float(sm_scale) if sm_scale else 0.0
    opts.num_cus = int(num_cus)
    opts.max_splits = int(max_splits)
    opts.min_chunk = int(min_chunk)
    opts.flags = ((AK_PLAN_HOST_ONLY if host_only else 0) |
                  (AK_PLAN_MERGE_IN_KERNEL if merge_in_kernel else 0) |
                  (AK_PLAN_SHARED_PAGES if shared_pages else 0) |
                  (AK_PLAN_STREAM_K if stream_k else 0))
    opts.stream = None if host_only else _stream_ptr(stream)
    idx_ptr = None
    if kv_indices is not None:
        if not host_only:
            import torch

            if kv_indices.dtype != torch.int32 or not kv_indices.is_contiguous():
                raise TypeError("kv_indices must be a contiguous int32 device tensor")
            idx_ptr = ctypes.c_void_p(kv_indices.data_ptr()) if kv_indices.numel() else None
    h = ctypes.c_void_p()
    _check(_lib.ak_plan(qo_p, kv_p, idx_ptr, last_p, R, num_qo_heads, num_kv_heads, head_dim,
                        page_size, int(bool(causal)), int(window), ctypes.byref(opts),
                        ctypes.byref(h)))
    return Plan(h, num_qo_heads, num_kv_heads, head_dim, page_size, host_only, kv_indices)


def ak_plan_fixed(max_batch: int, max_tokens: int, kv_indices, num_qo_heads: int,
                  num_kv_heads: int, head_dim: int, page_size: int, causal: bool = True,
                  window: int = -1, sm_scale: float | None = None, num_cus: int = 0,
                  max_splits: int = 0, min_chunk: int = 0, host_only: bool = False,
                  max_pages: int | None = None, max_query_len: int = 0,
                  merge_in_kernel: bool = False, shared_pages: bool = False, stream_k: bool = False,
                  stream=None) -> Plan:
    """A plan with a fixed device workspace for graph capture.  kv_indices is the
    stable device int32 buffer later batches write their page ids into (its size
    is the page capacity); host-only plans take None and max_pages.  max_query_len
    bounds any one request's query tokens (0 = max_tokens; 1 for pure decode)."""
    opts = AkPlanOpts()
    opts.sm_scale = float(sm_scale) if sm_scale else 0.0
    opts.num_cus = int(num_cus)
    opts.max_splits = int(max_splits)
    opts.min_chunk = int(min_chunk)
    opts.flags = ((AK_PLAN_HOST_ONLY if host_only else 0) |
                  (AK_PLAN_MERGE_IN_KERNEL if merge_in_kernel else 0) |
                  (AK_PLAN_SHARED_PAGES if shared_pages else 0) |
                  (AK_PLAN_STREAM_K if stream_k else 0))
    opts.stream = None if host_only else _stream_ptr(stream)
    idx_ptr = None
    if kv_indices is not None and not host_only:
        import torch

        if kv_indices.dtype != torch.int32 or not kv_indices.is_contiguous():
            raise TypeError("kv_indices must be a contiguous int32 device tensor")
        idx_ptr = ctypes.c_void_p(kv_indices.data_ptr())
        if max_pages is None:
            max_pages = kv_indices.numel()
    h = ctypes.c_void_p()
    _check(_lib.ak_plan_fixed(int(max_batch), int(max_tokens), int(max_query_len),
                              int(max_pages or 0), idx_ptr,
                              num_qo_heads, num_kv_heads, head_dim, page_size, int(bool(causal)),
                              int(window), ctypes.byref(opts), ctypes.byref(h)))
    plan = Plan(h, num_qo_heads, num_kv_heads, head_dim, page_size, host_only, kv_indices)
    plan.fixed = True
    return plan


def ak_plan_update(plan: Plan, qo_indptr, kv_indptr, last_page_len, stream=None) -> None:
    """Plan a new batch into a fixed plan's workspace (host arrays as for ak_plan)."""
    qo, qo_p = _host_i32(qo_indptr)
    kv, kv_p = _host_i32(kv_indptr)
    last, last_p = _host_i32(last_page_len)
    R = len(qo) - 1
    if len(kv) != R + 1 or len(last) != R:
        raise ValueError("qo_indptr/kv_indptr need batch_size+1 entries, last_page_len batch_size")
    _check(_lib.ak_plan_update(plan.handle, qo_p, kv_p, last_p, R,
                               None if plan.host_only else _stream_ptr(stream)))


def ak_plan_destroy(plan: Plan) -> None:
    if plan is not None and plan.handle is not None and plan.handle.value:
        _lib.ak_plan_destroy(plan.handle)
        plan.handle = None


def ak_run(plan: Plan, q, k_cache, v_cache, out=None, lse=None, k_scale: float = 1.0,
           v_scale: float = 1.0, stream=None):
    """Attention for one layer; returns (out, lse).  out/lse are allocated if None
    (pass them to keep the call allocation-free)."""
    import torch

    if out is None:
        out = torch.empty_like(q)
    dq, dk, dv, do = (_desc(q), _desc(k_cache, k_scale), _desc(v_cache, v_scale),
                      _desc(out))
    dl = _desc(lse) if lse is not None else None
    _check(_lib.ak_run(plan.handle, ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv),
                       ctypes.byref(do), ctypes.byref(dl) if dl is not None else None,
                       _stream_ptr(stream)))
    return out, lse


def ak_run_noalloc(qo_indptr, kv_indptr, kv_indices, last_page_len, num_qo_heads: int,
                   num_kv_heads: int, head_dim: int, page_size: int, q, k_cache, v_cache, out, lse=None,
                   causal: bool = True, window: int = -1, k_scale: float = 1.0, v_scale: float = 1.0,
                   sm_scale: float | None = None, num_cus: int = 0, max_splits: int = 0,
                   min_chunk: int = 0, merge_in_kernel: bool = False, shared_pages: bool = False,
                   stream_k: bool = False, stream=None):
    """Plan and run one layer without any allocation by the library (its split
    workspace is a fixed device array); out (and lse) must be given."""
    qo, qo_p = _host_i32(qo_indptr)
    kv, kv_p = _host_i32(kv_indptr)
    last, last_p = _host_i32(last_page_len)
    R = len(qo) - 1
    if len(kv) != R + 1 or len(last) != R:
        raise ValueError("qo_indptr/kv_indptr need batch_size+1 entries, last_page_len batch_size")
    opts = AkPlanOpts()
    opts.sm_scale = float(sm_scale) if sm_scale else 0.0
    opts.num_cus = int(num_cus)
    opts.max_splits = int(max_splits)
    opts.min_chunk = int(min_chunk)
    opts.flags = ((AK_PLAN_MERGE_IN_KERNEL if merge_in_kernel else 0) |
                  (AK_PLAN_SHARED_PAGES if shared_pages else 0) |
                  (AK_PLAN_STREAM_K if stream_k else 0))
    idx_ptr = None
    if kv_indices is not None and kv_indices.numel():
        import torch

        if kv_indices.dtype != torch.int32 or not kv_indices.is_contiguous():
            raise TypeError("kv_indices must be a contiguous int32 device tensor")
        idx_ptr = ctypes.c_void_p(kv_indices.data_ptr())
    dq, dk, dv, do = (_desc(q), _desc(k_cache, k_scale), _desc(v_cache, v_scale), _desc(out))
    dl = _desc(lse) if lse is not None else None
    _check(_lib.ak_run_noalloc(qo_p, kv_p, idx_ptr, last_p, R, num_qo_heads, num_kv_heads,
                               head_dim, page_size, int(bool(causal)), int(window),
                               ctypes.byref(opts), ctypes.byref(dq), ctypes.byref(dk),
                               ctypes.byref(dv), ctypes.byref(do),
                               ctypes.byref(dl) if dl is not None else None, _stream_ptr(stream)))
    return out, lse


def ak_merge_states(o_a, lse_a, o_b, lse_b, out=None, lse_out=None, stream=None):
    """Combine two attention states over disjoint key sets of the same rows;
    returns (out, lse_out).  out / lse_out are allocated if None (out may be o_a
    or o_b for an in-place merge)."""
    import torch

    if out is None:
        out = torch.empty_like(o_a)
    if lse_out is None:
        lse_out = torch.empty_like(lse_a)
    da, dla, db, dlb, do, dlo = (_desc(o_a), _desc(lse_a), _desc(o_b),
                                 _desc(lse_b), _desc(out), _desc(lse_out))
    _check(_lib.ak_merge_states(ctypes.byref(da), ctypes.byref(dla), ctypes.byref(db),
                                ctypes.byref(dlb), ctypes.byref(do), ctypes.byref(dlo),
                                _stream_ptr(stream)))
    return out, lse_out


def ak_plan_info(plan: Plan) -> dict:
    buf = (ctypes.c_int64 * 13)()
    _check(_lib.ak_plan_info(plan.handle, buf, 13))
    keys = ["batch_size", "total_q", "items", "small_items", "large_items", "split_units",
            "merge_jobs", "partial_rows", "cap_small_items", "cap_large_items", "cap_merge_jobs",
            "cap_partial_rows", "stream_k_workgroups"]
    return dict(zip(keys, [int(x) for x in buf]))


def ak_plan_workgroups(plan: Plan) -> np.ndarray:
    """A stream-K plan's workgroup table wg_first (int32 [P + 1]; empty otherwise)."""
    n = ak_plan_info(plan)["stream_k_workgroups"]
    buf = np.zeros(max(n + 1, 1), dtype=np.int32)
    cnt = ctypes.c_int64()
    _check(_lib.ak_plan_workgroups(plan.handle, buf.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                   len(buf), ctypes.byref(cnt)))
    return buf[:cnt.value]


def ak_plan_export(plan: Plan):
    """Returns (items int32 [n, 8], kv_lens int32 [batch_size])."""
    info = ak_plan_info(plan)
    n = info["items"]
    items = np.zeros((max(n, 1), 8), dtype=np.int32)
    lens = np.zeros(max(info["batch_size"], 1), dtype=np.int32)
    cnt = ctypes.c_int64()
    _check(_lib.ak_plan_export(plan.handle, items.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                               n, ctypes.byref(cnt),
                               lens.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))))
    return items[:n], lens[:info["batch_size"]]


def ak_gather_slots(plan: Plan, slots, addressing: int = 0, stream=None) -> None:
    """Write every request's KV slots (device int64 tensor of sum L entries) through
    the decode kernels' (addressing 0) or the prefill kernels' row addressing (1; 2 for
    its 32-bit form)."""
    _check(_lib.ak_gather_slots(plan.handle, int(addressing), ctypes.c_void_p(slots.data_ptr()),
                                _stream_ptr(stream)))


def _dev_i32_matrix(t, name):
    if t.dtype != _torch().int32 or t.dim() != 2 or not t.is_contiguous() or not t.is_cuda:
        raise AkError(-1, f"{name}: expected a contiguous device int32 [rows, cols] tensor")
    return t


def _dev_i32_vector(t, n, name):
    if t.dtype != _torch().int32 or t.dim() != 1 or t.numel() < n or not t.is_cuda:
        raise AkError(-1, f"{name}: expected a device int32 vector of at least {n} entries")
    return t


def _torch():
    import torch

    return torch


def ak_csr_from_block_table(block_table, seq_lens, page_size: int, kv_indices=None,
                            kv_indptr=None, last_page_len=None, block_ratio: int = 1, stream=None):
    """Build (kv_indptr, kv_indices, last_page_len) from a device block table
    [R, max_blocks] and device seq_lens [R] (all int32).  With block_ratio > 1 the
    table holds manager blocks of block_ratio * page_size tokens and the CSR lists
    page_size-token kernel pages.  kv_indices defaults to R * max_blocks *
    block_ratio entries, enough for any lengths; the valid prefix is
    kv_indices[:kv_indptr[R]]."""
    torch = _torch()
    _dev_i32_matrix(block_table, "block_table")
    R, max_blocks = block_table.shape
    _dev_i32_vector(seq_lens, R, "seq_lens")
    dev = block_table.device
    if kv_indptr is None:
        kv_indptr = torch.empty(R + 1, dtype=torch.int32, device=dev)
    if last_page_len is None:
        last_page_len = torch.empty(R, dtype=torch.int32, device=dev)
    if kv_indices is None:
        kv_indices = torch.empty(max(R * max_blocks * int(block_ratio), 1), dtype=torch.int32,
                                 device=dev)
    _dev_i32_vector(kv_indptr, R + 1, "kv_indptr")
    _dev_i32_vector(last_page_len, R, "last_page_len")
    _dev_i32_vector(kv_indices, 0, "kv_indices")
    _check(_lib.ak_csr_from_block_table(
        ctypes.c_void_p(block_table.data_ptr()), max_blocks, ctypes.c_void_p(seq_lens.data_ptr()),
        R, int(page_size), int(block_ratio), ctypes.c_void_p(kv_indptr.data_ptr()),
        ctypes.c_void_p(kv_indices.data_ptr()), kv_indices.numel(),
        ctypes.c_void_p(last_page_len.data_ptr()), _stream_ptr(stream)))
    return kv_indptr, kv_indices, last_page_len


def ak_slot_mapping(block_table, qo_indptr, seq_lens, page_size: int, num_tokens=None, out=None,
                    stream=None):
    """Slots of every new token (device int64 [num_tokens]; -1 for padding) from a
    device block table [R, max_pages], qo_indptr [R + 1] and seq_lens [R] (int32).
    num_tokens defaults to the batch's token count, which costs a device read."""
    torch = _torch()
    _dev_i32_matrix(block_table, "block_table")
    R, max_pages = block_table.shape
    _dev_i32_vector(qo_indptr, R + 1, "qo_indptr")
    _dev_i32_vector(seq_lens, R, "seq_lens")
    if out is None:
        if num_tokens is None:
            num_tokens = int(qo_indptr[R].item())
        out = torch.empty(num_tokens, dtype=torch.int64, device=block_table.device)
    if out.dtype != torch.int64 or not out.is_contiguous() or not out.is_cuda:
        raise AkError(-1, "slot_mapping: expected a contiguous device int64 tensor")
    _check(_lib.ak_slot_mapping(
        ctypes.c_void_p(block_table.data_ptr()), max_pages, ctypes.c_void_p(qo_indptr.data_ptr()),
        ctypes.c_void_p(seq_lens.data_ptr()), R, int(page_size), ctypes.c_void_p(out.data_ptr()),
        out.numel(), _stream_ptr(stream)))
    return out


KERNEL_KINDS = ["store_kv", "attn_small", "attn_large", "merge", "attn_f32"]


def ak_profile_enable(on: bool = True, kinds=None) -> None:
    """Time launches with HIP events: every kernel kind, or only the named ones
    (names from KERNEL_KINDS)."""
    mask = 0
    if on:
        mask = AK_PROFILE_ALL if kinds is None else sum(1 << KERNEL_KINDS.index(k) for k in kinds)
    _check(_lib.ak_profile_enable(mask))


def ak_profile_read() -> dict:
    n = len(KERNEL_KINDS)
    launches = (ctypes.c_int64 * n)()
    ms = (ctypes.c_double * n)()
    _check(_lib.ak_profile_read(launches, ms, n))
    return {k: (int(launches[i]), float(ms[i])) for i, k in enumerate(KERNEL_KINDS)}


def ak_fp8_to_bf16(codes, out=None, stream=None):
    """Widen device uint8 E4M3 codes (numel a multiple of 8) to bf16 with the
    kernels' conversion; returns a bfloat16 tensor."""
    import torch

    if out is None:
        out = torch.empty(codes.shape, dtype=torch.bfloat16, device=codes.device)
    _check(_lib.ak_fp8_to_bf16(ctypes.c_void_p(codes.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                               codes.numel(), _stream_ptr(stream)))
    return out
