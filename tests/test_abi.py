"""The C-ABI library loads and exports every symbol include/ak.h declares (no GPU)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "ak.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ak_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("ak_store_kv", "ak_plan", "ak_run", "ak_plan_destroy", "ak_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol():
    import paged_kv_attention_store_amd as ak

    lib = ctypes.CDLL(ak.LIB_PATH)
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing
    assert set(ak.EXPORTED) == set(_declared())


def test_version_and_error_text():
    import paged_kv_attention_store_amd as ak

    assert "gfx950" in ak.ak_version()
    assert isinstance(ak.ak_last_error(), str)


def test_binding_struct_layout_matches_header():
    import paged_kv_attention_store_amd as ak

    # ak_tensor: void* + 2*int32 + 4*int64 + 4*int64 + float (+ padding) = 88 bytes
    assert ctypes.sizeof(ak.AkTensor) == 88
    assert ctypes.sizeof(ak.AkPlanOpts) == 32


def test_one_hip_runtime_per_process():
    # torch loads its own HIP runtime by path; the binding must make libak share
    # it whatever the import order, or kernels launch on a runtime without devices
    import subprocess
    import sys

    code = ("import paged_kv_attention_store_amd, torch\n"
            "libs = {l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}\n"
            "print(len(libs))\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip().splitlines()[-1] == "1"


def test_cached_descriptors_match_fresh_ones():
    # the entry points reuse descriptors keyed by everything a descriptor holds;
    # for any tensor the cached one equals a freshly built one field by field
    import torch

    import paged_kv_attention_store_amd as ak

    base = torch.zeros(6, 4, 8, 16, dtype=torch.bfloat16)
    views = [base, base[:, :2], base[1:], base.permute(1, 0, 2, 3), base[..., :8],
             base.view(24, 8, 16), torch.zeros(0, 3, dtype=torch.float32),
             torch.zeros(5, dtype=torch.int64)]
    for _ in range(2):                        # second pass: served from the cache
        for v in views:
            for scale in (1.0, 0.5):
                a, b = ak._desc(v, scale), ak.tensor_desc(v, scale)
                assert bytes(a) == bytes(b)
    # a new tensor at a reused address with other strides gets its own descriptor
    x = torch.zeros(8, 8)
    d1 = bytes(ak._desc(x))
    y = x.t()
    assert bytes(ak._desc(y)) != d1 and bytes(ak._desc(y)) == bytes(ak.tensor_desc(y))
