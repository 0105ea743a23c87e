"""CPU tests of the C ABI: the library loads, exports every function that
include/w4.h declares, and rejects bad arguments on the host before touching
the GPU (these calls return before any HIP call is made)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    with open(os.path.join(ROOT, "include", "w4.h")) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(w4_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def w4():
    import weight_only_bit_unpack_amd as m
    return m


def test_header_declares_the_calls():
    names = _declared()
    for n in ["w4_quantize_pack", "w4_unpack_dequant", "w4_gemv", "w4_gemm", "w4_linear", "w4_lut16_fit",
              "w4_signmag8_fit", "w4_signmag8_fit_warm", "w4_quantize_dyadic5",
              "w4_gemv_batched_plan", "w4_gemv_batched", "w4_status_str", "w4_group_size"]:
        assert n in names


def test_library_exports_every_declared_symbol(w4):
    lib = ctypes.CDLL(w4.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name
    assert set(_declared()) == set(w4.EXPORTED)


def test_group_sizes_and_status_strings(w4):
    assert [w4.w4_group_size(c) for c in (0, 1, 2, 3, 4, 5, 6, 7)] == [64, 64, 32, 64, 64, 64, 64, -1]
    for s in range(6):
        assert w4.w4_status_str(s).startswith("W4_")


def _gemv(w4, codec=0, n=16, k=64, packed=16, scales=16, cb=16, x=16, m=1, y=16, yd=0,
          fn="w4_gemv"):
    P = lambda v: None if v is None else ctypes.c_void_p(v)
    return getattr(w4._lib, fn)(codec, n, k, P(packed), P(scales), P(cb), P(x), m, P(y), yd, None)


def test_validation_errors(w4):
    E = {"inval": 1, "shape": 2, "align": 3, "unsup": 4}
    assert _gemv(w4, codec=7) == E["inval"]
    assert _gemv(w4, n=-1) == E["inval"]
    assert _gemv(w4, k=96) == E["shape"]
    assert _gemv(w4, m=17) == E["shape"]
    assert _gemv(w4, m=-1) == E["inval"]
    assert _gemv(w4, packed=None) == E["inval"]
    assert _gemv(w4, packed=8) == E["align"]
    assert _gemv(w4, scales=None) == E["inval"]
    assert _gemv(w4, scales=17) == E["align"]
    assert _gemv(w4, codec=1, cb=None) == E["inval"]
    assert _gemv(w4, codec=3, cb=None) == E["inval"]
    assert _gemv(w4, codec=3, scales=None) == E["inval"]
    assert _gemv(w4, codec=3, cb=24) == E["align"]
    assert _gemv(w4, codec=4, cb=None) == E["inval"]
    assert _gemv(w4, codec=4, scales=None) == E["inval"]
    assert _gemv(w4, codec=4, cb=24) == E["align"]
    assert _gemv(w4, codec=2, scales=None, cb=32 + 8) == E["align"]
    assert _gemv(w4, x=None) == E["inval"]
    assert _gemv(w4, x=24) == E["align"]
    assert _gemv(w4, y=None) == E["inval"]
    assert _gemv(w4, y=18) == E["align"]
    assert _gemv(w4, yd=2) == E["unsup"]
    # k beyond W4_MAX_MATMUL_K (4,194,304) is rejected before any launch
    assert _gemv(w4, k=4194304 + 64) == E["shape"]
    assert _gemv(w4, k=4194304 + 64, fn="w4_gemm") == E["shape"]
    # w4_linear validates as the call it selects
    assert _gemv(w4, m=-1, fn="w4_linear") == E["inval"]
    assert _gemv(w4, m=17, packed=8, fn="w4_linear") == E["align"]
    assert _gemv(w4, k=96, fn="w4_linear") == E["shape"]
    # empty problems are accepted without touching anything
    assert _gemv(w4, n=0, packed=None, scales=None, x=None, y=None) == 0
    assert _gemv(w4, m=0, x=None, y=None) == 0


def test_quantize_dequant_validation(w4):
    q = w4._lib.w4_quantize_pack
    d = w4._lib.w4_unpack_dequant
    P = ctypes.c_void_p
    assert q(0, 4, 100, P(16), P(16), P(16), None, None) == 2
    assert q(0, 4, 64, None, P(16), P(16), None, None) == 1
    assert q(0, 4, 64, P(8), P(16), P(16), None, None) == 3
    assert q(0, 0, 64, None, None, None, None, None) == 0
    assert d(1, 4, 64, P(16), P(16), None, P(16), None) == 1
    assert d(0, 4, 64, P(16), P(16), None, None, None) == 1
    assert d(0, 4, 64, P(16), P(16), None, P(8), None) == 3


def test_lut16_fit_validation(w4):
    f = w4._lib.w4_lut16_fit
    P = ctypes.c_void_p
    ok = dict(n=4, k=64, w=P(16), s=P(16), L=P(16), it=25)
    call = lambda **kw: f(*[{**ok, **kw}[a] for a in ("n", "k", "w", "s", "L", "it")], None)
    assert call(n=-1) == 1
    assert call(k=96) == 2
    assert call(it=-1) == 1
    assert call(it=1025) == 1
    assert call(w=None) == 1 and call(s=None) == 1 and call(L=None) == 1
    assert call(w=P(8)) == 3 and call(L=P(24)) == 3 and call(s=P(17)) == 3
    assert call(n=0, w=None, s=None, L=None) == 0
    assert call(k=0, w=None, s=None, L=None) == 0
    assert call(n=1 << 35, k=128) == 2          # 2^36 groups: more than 16 * (2^31 - 1)


def test_signmag8_fit_validation(w4):
    f = w4._lib.w4_signmag8_fit
    P = ctypes.c_void_p
    ok = dict(n=4, k=32, w=P(16), cb=P(16), it=25)
    call = lambda **kw: f(*[{**ok, **kw}[a] for a in ("n", "k", "w", "cb", "it")], None)
    assert call(n=-1) == 1 and call(k=-32) == 1
    assert call(k=48) == 2
    assert call(it=-1) == 1 and call(it=1025) == 1
    assert call(w=None) == 1 and call(cb=None) == 1
    assert call(w=P(8)) == 3 and call(cb=P(24)) == 3
    assert call(n=0, w=None, cb=None) == 0
    assert call(k=0, w=None, cb=None) == 0
    assert call(n=1 << 36, k=64) == 2          # 2^37 groups: more than 32 * (2^31 - 1)


def test_signmag8_fit_warm_validation(w4):
    f = w4._lib.w4_signmag8_fit_warm
    P = ctypes.c_void_p
    ok = dict(n=4, k=32, w=P(16), cb=P(16), pr=None, it=25)
    call = lambda **kw: f(*[{**ok, **kw}[a] for a in ("n", "k", "w", "cb", "pr", "it")], None)
    assert call(n=-1) == 1 and call(k=-32) == 1
    assert call(k=48) == 2
    assert call(it=-1) == 1 and call(it=1025) == 1
    assert call(w=None) == 1 and call(cb=None) == 1
    assert call(w=P(8)) == 3 and call(cb=P(24)) == 3
    assert call(n=0, w=None, cb=None) == 0
    assert call(k=0, w=None, cb=None) == 0
    assert call(n=1 << 33, k=64) == 2          # 2^34 groups: more than 2 * (2^31 - 1)


def test_quantize_dyadic5_validation(w4):
    f = w4._lib.w4_quantize_dyadic5
    P = ctypes.c_void_p
    ok = dict(n=4, k=64, w=P(16), wd=None, p=P(16), m=P(16), s=P(16))
    call = lambda **kw: f(*[{**ok, **kw}[a] for a in ("n", "k", "w", "wd", "p", "m", "s")], None)
    assert call(n=-1) == 1 and call(k=-64) == 1
    assert call(k=96) == 2
    assert call(w=None) == 1 and call(p=None) == 1 and call(m=None) == 1 and call(s=None) == 1
    assert call(w=P(8)) == 3 and call(p=P(8)) == 3 and call(m=P(4)) == 3 and call(s=P(3)) == 3
    assert call(n=0, w=None, p=None, m=None, s=None) == 0
    # the generic quantize call does not write DYADIC5's second plane
    assert w4._lib.w4_quantize_pack(4, 4, 64, P(16), P(16), P(16), P(16), None) == 4


def test_struct_sizes_match_the_header(w4):
    assert ctypes.sizeof(w4.W4Problem) == 64
    assert ctypes.sizeof(w4.W4BatchInfo) == 40


def test_batched_plan_validation(w4):
    arr = (w4.W4Problem * 3)()
    for i in range(2):
        arr[i] = w4.W4Problem(16, 16, None, 16, 16, 100 + 64 * i, 128 + 64 * i, 0)
    arr[2] = w4.W4Problem(8, 8, 8, 8, 8, 7, 7, 7)   # past count: never touched
    info = w4.W4BatchInfo()
    plan = lambda m: w4._lib.w4_gemv_batched_plan(0, m, 0, arr, 2, ctypes.byref(info))
    # m = 16: 64-row blocks; largest k first: problem 1 (k = 192, 3 blocks) gets
    # blocks 0..2, problem 0 blocks 3..4
    assert plan(16) == 0
    assert info.total_tiles == 2 + 3 and arr[1].tile_begin == 0 and arr[0].tile_begin == 3
    assert (info.k_min, info.k_max, info.count, info.m) == (128, 192, 2, 16)
    assert (arr[2].n, arr[2].k, arr[2].tile_begin) == (7, 7, 7)
    assert info.tile_rows == 64
    # m = 1 with few tiles: 16-row tiles (7 + 11), the same order
    assert plan(1) == 0 and info.m == 1 and info.tile_rows == 16
    assert info.total_tiles == 7 + 11 and arr[1].tile_begin == 0 and arr[0].tile_begin == 11
    assert w4._lib.w4_gemv_batched(0, 2, 0, ctypes.c_void_p(16), ctypes.byref(info), None) == 1
    arr[1].k = 100
    assert plan(1) == 2
    assert plan(17) == 2
    assert w4._lib.w4_gemv_batched(0, 1, 0, ctypes.c_void_p(8), ctypes.byref(info), None) == 3
    bad = w4.W4BatchInfo(5, -1, 128, 2, 1, 64, 0)
    assert w4._lib.w4_gemv_batched(0, 1, 0, ctypes.c_void_p(16), ctypes.byref(bad), None) == 1
    odd_rows = w4.W4BatchInfo(5, 128, 192, 2, 1, 48, 0)
    assert w4._lib.w4_gemv_batched(0, 1, 0, ctypes.c_void_p(16), ctypes.byref(odd_rows), None) == 1
    m16_rows = w4.W4BatchInfo(5, 128, 192, 2, 16, 16, 0)     # 16-row tiles only for m = 1
    assert w4._lib.w4_gemv_batched(0, 16, 0, ctypes.c_void_p(16), ctypes.byref(m16_rows), None) == 1
    empty = w4.W4BatchInfo(0, 0, 0, 0, 1)
    assert w4._lib.w4_gemv_batched(0, 1, 0, None, ctypes.byref(empty), None) == 0


def test_signmag8_group_rule(w4):
    """SIGNMAG8 takes k a multiple of its group of 32 in quantize and dequant
    (a null buffer then is the first error), but the matrix calls need 64."""
    E = {"inval": 1, "shape": 2}
    P = ctypes.c_void_p
    assert w4._lib.w4_quantize_pack(2, 4, 96, None, None, None, None, None) == E["inval"]
    assert w4._lib.w4_unpack_dequant(2, 4, 96, None, None, None, None, None) == E["inval"]
    assert w4._lib.w4_quantize_pack(2, 4, 80, None, None, None, None, None) == E["shape"]
    assert w4._lib.w4_quantize_pack(0, 4, 96, None, None, None, None, None) == E["shape"]
    assert _gemv(w4, codec=2, k=96, scales=None) == E["shape"]
    assert _gemv(w4, codec=2, k=96, scales=None, fn="w4_gemm") == E["shape"]


def test_batched_flags_checked(w4):
    """w4_gemv_batched rejects an info record whose flags hold bits the plan
    never writes, and a ragged plan launched as W4_LUT16S_IL (before any
    launch)."""
    info = w4.W4BatchInfo(total_tiles=1, k_min=64, k_max=64, count=1, m=1, tile_rows=64, flags=2)
    assert w4._lib.w4_gemv_batched(0, 1, 0, ctypes.c_void_p(16), ctypes.byref(info), None) == 1
    # a plan with a k that is not a multiple of 256 (bit 0) cannot run as the
    # interleaved LUT16S layout, whose records are whole 256-k blocks
    ragged = w4.W4BatchInfo(total_tiles=1, k_min=64, k_max=64, count=1, m=1, tile_rows=64,
                            flags=1)
    assert w4._lib.w4_gemv_batched(6, 1, 0, ctypes.c_void_p(16), ctypes.byref(ragged), None) == 2


def test_lut16s_variants_rules(w4):
    """W4_LUT16S_PERM takes LUT16S's side data everywhere; W4_LUT16S_IL needs k
    a multiple of 256 and a codebook, no scales, and only the GEMV takes it;
    w4_lut16s_interleave validates like the other layout calls."""
    E = {"inval": 1, "shape": 2, "unsup": 4}
    assert _gemv(w4, codec=5, scales=None) == E["inval"]
    assert _gemv(w4, codec=5, cb=None) == E["inval"]
    assert _gemv(w4, codec=6, k=192, scales=None) == E["shape"]
    assert _gemv(w4, codec=6, k=256, scales=None, cb=None) == E["inval"]
    assert _gemv(w4, codec=6, k=256, scales=None, fn="w4_gemm") == E["unsup"]
    assert w4._lib.w4_quantize_pack(6, 4, 256, ctypes.c_void_p(16), ctypes.c_void_p(16), None,
                                    ctypes.c_void_p(16), None) == E["unsup"]
    assert w4._lib.w4_unpack_dequant(6, 4, 256, ctypes.c_void_p(16), None, ctypes.c_void_p(16),
                                     ctypes.c_void_p(16), None) == E["unsup"]
    assert w4._lib.w4_lut16s_interleave(4, 192, None, None, None, None) == E["shape"]
    assert w4._lib.w4_lut16s_interleave(4, 256, None, None, None, None) == E["inval"]
    assert w4._lib.w4_lut16s_interleave(-1, 256, None, None, None, None) == E["inval"]


def test_binding_rejects_host_tensors(w4):
    """The Python binding checks its tensors before calling the library: a
    tensor in host memory is refused with ValueError (no GPU is touched)."""
    import torch
    packed = torch.zeros((4, 32), dtype=torch.uint8)
    scales = torch.zeros((4, 1), dtype=torch.bfloat16)
    x = torch.zeros((1, 64), dtype=torch.bfloat16)
    for fn in (w4.w4_gemv, w4.w4_gemm, w4.w4_linear):
        with pytest.raises(ValueError, match="packed must be a CUDA"):
            fn(packed, x, w4.W4_DYADIC, scales=scales)
    with pytest.raises(ValueError, match="w must be a CUDA"):
        w4.w4_quantize_pack(torch.zeros((4, 64), dtype=torch.bfloat16), w4.W4_DYADIC)
    with pytest.raises(ValueError, match="packed is required"):
        w4.w4_gemv(None, x, w4.W4_DYADIC, scales=scales)
