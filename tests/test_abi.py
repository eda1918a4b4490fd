"""The C-ABI library loads and exports every symbol include/*.h declares.

CPU only: no call here touches a GPU (only the host-only size and error-text
entry points are called, and entry points with arguments their host checks
reject before anything is launched).
"""
import ctypes
import glob
import os
import re
import subprocess

import pytest

import moe_expert_load_amd as mx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _ensure_built():
    if not os.path.exists(mx.LIB_PATH):
        from moe_expert_load_amd import build
        build.build()


def declared_entry_points():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?\w+\s*\**\s*(moe_\w+)\s*\(", text, re.M):
            names.add(m.group(1))
    return names


def test_header_declares_the_entry_points():
    names = declared_entry_points()
    assert names == set(mx.ENTRY_POINTS)


def test_library_exports_every_declared_symbol():
    _ensure_built()
    lib = ctypes.CDLL(mx.LIB_PATH)
    for name in declared_entry_points():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", mx.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (moe_\w+)", out))
    assert declared_entry_points() <= exported


def test_host_only_calls_and_validation():
    _ensure_built()
    cfg = mx.make_cfg(8, 8192, 384, 8, 7168, 2048, 48)
    sizes = mx.moe_plan_sizes(cfg)
    assert sizes[0] == 4 * 384 and sizes[1] == 4 * 8
    assert sizes[2] == 4 * 8 * 8192 * 8
    assert sizes[3] == 4 * 8 * (384 + 48 + 1)
    assert sizes[7] == 16 * (384 + 8 - 1) and sizes[8] == 16
    assert sizes[9] > 0
    assert mx.moe_gemm_workspace_size(cfg) > 0
    bad = [
        mx.make_cfg(8, 16, 30, 2, 128, 64, 3),            # E % R != 0
        mx.make_cfg(4, 16, 8, 9, 128, 64, 2),             # K > E
        mx.make_cfg(4, 16, 8, 2, 128, 64, 1),             # train needs B = E/R
        mx.make_cfg(4, 16, 8, 2, 128, 64, 3, mx.MODE_INFER),  # B > E/R
        mx.make_cfg(4, 16, 8, 2, 100, 64, 2),             # H % 8 != 0
        mx.make_cfg(4, 16, 8, 2, 128, 64, 2, 7),          # bad mode
    ]
    for c in bad:
        with pytest.raises(mx.MoeError) as ei:
            mx.moe_plan_sizes(c)
        assert ei.value.code == mx.MOE_EINVAL
    with pytest.raises(mx.MoeError) as ei:
        mx.moe_plan_sizes(mx.make_cfg(4, 16, 4096, 2, 128, 64, 1024))
    assert ei.value.code == mx.MOE_ELIMIT
    with pytest.raises(mx.MoeError) as ei:
        mx.moe_plan_sizes(mx.make_cfg(64, 1 << 20, 896, 64, 128, 64, 14))
    assert ei.value.code == mx.MOE_ELIMIT
    # tokens: R*S < 2^24 (one 256-thread workgroup per token in dispatch)
    mx.moe_plan_sizes(mx.make_cfg(1024, (1 << 14) - 1, 1024, 1, 8, 8, 1))
    with pytest.raises(mx.MoeError) as ei:
        mx.moe_plan_sizes(mx.make_cfg(1024, 1 << 14, 1024, 1, 8, 8, 1))
    assert ei.value.code == mx.MOE_ELIMIT
    # inference may use fewer slots, even none
    mx.moe_plan_sizes(mx.make_cfg(8, 8192, 384, 8, 7168, 2048, 4, mx.MODE_INFER))
    mx.moe_plan_sizes(mx.make_cfg(8, 8192, 384, 8, 7168, 2048, 0, mx.MODE_INFER))
    # SwiGLU entry points: host checks come before any launch
    lib = mx.load()
    big = mx.make_cfg(8, 16, 8, 2, 65536, 16384, 1)        # H * H' * 4 = 2^32
    assert lib.moe_grouped_gemm_swiglu(ctypes.byref(big), None, None, None, None, None, None,
                                       0, 8, None, None) == mx.MOE_ELIMIT
    small = mx.make_cfg(4, 16, 8, 2, 128, 64, 2)
    assert lib.moe_grouped_gemm_swiglu(ctypes.byref(small), None, None, None, None, None, None,
                                       0, 4, None, None) == mx.MOE_EINVAL
    assert lib.moe_grouped_gemm_swiglu(ctypes.byref(small), None, None, None, None, None, None,
                                       2, 2, None, None) == mx.MOE_OK      # empty rank range
    assert lib.moe_grouped_gemm_swiglu(ctypes.byref(small), None, None, None, None, None, None,
                                       0, 5, None, None) == mx.MOE_EINVAL
    assert lib.moe_swiglu_backward(ctypes.byref(small), None, None, None, None) == mx.MOE_EINVAL
    a, b = ctypes.c_void_p(1 << 20), ctypes.c_void_p((1 << 20) + 64)
    # d act overlapping dh13, and a misaligned pointer, are rejected
    assert lib.moe_swiglu_backward(ctypes.byref(small), ctypes.c_void_p(1 << 30), a, b,
                                   None) == mx.MOE_EINVAL
    assert lib.moe_swiglu_backward(ctypes.byref(small), ctypes.c_void_p((1 << 30) + 8),
                                   ctypes.c_void_p(1 << 24), ctypes.c_void_p(1 << 28),
                                   None) == mx.MOE_EINVAL
    # tensor bases off a 16-byte boundary are rejected before any launch
    A, M = ctypes.c_void_p(1 << 20), ctypes.c_void_p((1 << 20) + 8)
    fake = mx.moe_plan(*[ctypes.c_void_p(1 << 24) for _ in mx.PLAN_FIELDS])
    assert lib.moe_dispatch(ctypes.byref(small), ctypes.byref(fake), M, A, None) == mx.MOE_EINVAL
    assert lib.moe_combine(ctypes.byref(small), ctypes.byref(fake), A, A, M, None) == mx.MOE_EINVAL
    assert lib.moe_prefetch_weight(ctypes.byref(small), ctypes.byref(fake), A, M,
                                   None) == mx.MOE_EINVAL
    assert lib.moe_grouped_gemm(ctypes.byref(small), M, A, A, A, A, 0, 4, A,
                                None) == mx.MOE_EINVAL
    assert lib.moe_grouped_gemm_dgrad(ctypes.byref(small), A, A, A, A, M, 0, 4, A,
                                      None) == mx.MOE_EINVAL
    assert lib.moe_grouped_gemm_wgrad(ctypes.byref(small), ctypes.byref(fake), A, A, M, A, A,
                                      None) == mx.MOE_EINVAL
    assert lib.moe_grouped_gemm_swiglu(ctypes.byref(small), A, A, A, A, A, M, 0, 4, A,
                                       None) == mx.MOE_EINVAL
    assert lib.moe_reduce_grad(ctypes.byref(small), ctypes.byref(fake), A, M,
                               None) == mx.MOE_EINVAL
    assert mx.moe_strerror(mx.MOE_EINVAL).startswith("invalid")
    assert mx.moe_strerror(12345) == "unknown error code"


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError, match="not built"):
        mx.load(str(tmp_path / "nope.so"))
