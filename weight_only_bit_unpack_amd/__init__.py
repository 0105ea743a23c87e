"""Python binding of libw4, the gfx950 group-wise 4-bit weight library.

Argument marshalling only: every call checks device / dtype / shape of the
torch tensors, allocates outputs with torch when the caller passes none, and
forwards raw device pointers and the current HIP stream to the C ABI
(``include/w4.h``), whose functions carry the same names.  All computation
happens in the HIP kernels; there is no fallback of any kind, and importing
this package fails if ``libw4.so`` has not been built
(``python weight_only_bit_unpack_amd/build.py``).
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libw4.so")

W4_DYADIC, W4_LUT16, W4_SIGNMAG8, W4_LUT16S, W4_DYADIC5 = 0, 1, 2, 3, 4
W4_LUT16S_PERM, W4_LUT16S_IL = 5, 6
W4_F32, W4_BF16, W4_F16 = 0, 1, 2
GROUP = {W4_DYADIC: 64, W4_LUT16: 64, W4_SIGNMAG8: 32, W4_LUT16S: 64, W4_DYADIC5: 64,
         W4_LUT16S_PERM: 64, W4_LUT16S_IL: 64}
IL_RECORD = 144  # bytes of one W4_LUT16S_IL record (256 weights)

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python weight_only_bit_unpack_amd/build.py`")

_lib = ctypes.CDLL(LIB_PATH)
_P, _I32, _I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64


class W4Problem(ctypes.Structure):
    """Mirror of ``w4_gemv_problem``."""
    _fields_ = [("packed", _P), ("scales", _P), ("codebook", _P), ("x", _P), ("y", _P),
                ("n", _I64), ("k", _I64), ("tile_begin", _I64)]


class W4BatchInfo(ctypes.Structure):
    """Mirror of ``w4_gemv_batch_info``."""
    _fields_ = [("total_tiles", _I64), ("k_min", _I64), ("k_max", _I64), ("count", _I32),
                ("m", _I32), ("tile_rows", _I32), ("flags", _I32)]


_SIGS = {
    "w4_status_str": ([_I32], ctypes.c_char_p),
    "w4_group_size": ([_I32], _I32),
    "w4_quantize_pack": ([_I32, _I64, _I64, _P, _P, _P, _P, _P], _I32),
    "w4_unpack_dequant": ([_I32, _I64, _I64, _P, _P, _P, _P, _P], _I32),
    "w4_lut16_fit": ([_I64, _I64, _P, _P, _P, _I32, _P], _I32),
    "w4_signmag8_fit": ([_I64, _I64, _P, _P, _I32, _P], _I32),
    "w4_signmag8_fit_warm": ([_I64, _I64, _P, _P, _P, _I32, _P], _I32),
    "w4_quantize_dyadic5": ([_I64, _I64, _P, _P, _P, _P, _P, _P], _I32),
    "w4_lut16s_interleave": ([_I64, _I64, _P, _P, _P, _P], _I32),
    "w4_gemv": ([_I32, _I64, _I64, _P, _P, _P, _P, _I32, _P, _I32, _P], _I32),
    "w4_gemm": ([_I32, _I64, _I64, _P, _P, _P, _P, _I32, _P, _I32, _P], _I32),
    "w4_gemm_noalloc": ([_I32, _I64, _I64, _P, _P, _P, _P, _I32, _P, _I32, _P], _I32),
    "w4_linear": ([_I32, _I64, _I64, _P, _P, _P, _P, _I32, _P, _I32, _P], _I32),
    "w4_gemv_batched_plan": ([_I32, _I32, _I32, ctypes.POINTER(W4Problem), _I32,
                              ctypes.POINTER(W4BatchInfo)], _I32),
    "w4_gemv_batched": ([_I32, _I32, _I32, _P, ctypes.POINTER(W4BatchInfo), _P], _I32),
}
for _name, (_args, _res) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.argtypes = _args
    _fn.restype = _res

EXPORTED = tuple(_SIGS)


class W4Error(RuntimeError):
    def __init__(self, status):
        self.status = status
        super().__init__(_lib.w4_status_str(status).decode())


def _check(status):
    if status != 0:
        raise W4Error(status)


def w4_status_str(status):
    return _lib.w4_status_str(status).decode()


def w4_group_size(codec):
    return _lib.w4_group_size(codec)


# ------------------------------------------------------------------ marshalling
_U16 = (torch.bfloat16, torch.float16, torch.int16, torch.uint16)


# (the declared argtypes let ctypes take plain ints for the pointer arguments)
def _ptr(t):
    return None if t is None else t.data_ptr()


# The current stream's handle without building a Stream object (which costs
# a few microseconds per call), where this torch build has the query.
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream, dev=None):
    """HIP stream handle: the given torch stream, else the current stream of
    device dev (default: the current device)."""
    if stream is not None:
        return stream.cuda_stream
    if _raw_stream is None:
        return torch.cuda.current_stream().cuda_stream
    return _raw_stream(torch.cuda.current_device() if dev is None else dev)


def _need(t, name, dtypes, shape=None, dev=None):
    """Checks a tensor argument; dev: the current device's index when the
    caller already has it (a small call's checks cost more than its kernel)."""
    if t is None:
        raise ValueError(f"{name} is required")
    d = t.get_device()
    if d < 0:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if dev is None:
        dev = torch.cuda.current_device()
    if d != dev:
        raise ValueError(f"{name} is on {t.device}; the library works on the current device "
                         f"(cuda:{dev})")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and t.shape != shape:
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _k_of(codec, packed):
    """k of a quantized weight from its packed array's shape."""
    if codec == W4_LUT16S_IL:
        return packed.shape[1] // IL_RECORD * 256
    return 2 * packed.shape[1]


def _side_tables(codec, n, k, scales, codebook, dev=None):
    g = GROUP[codec]
    if codec in (W4_DYADIC, W4_LUT16, W4_LUT16S, W4_DYADIC5, W4_LUT16S_PERM):
        _need(scales, "scales", _U16, (n, k // 64), dev)
    if codec == W4_DYADIC5:
        _need(codebook, "codebook (high-bit plane)", (torch.uint8,), (n, k // 8), dev)
    if codec == W4_LUT16:
        _need(codebook, "codebook", _U16, (n, k // 64, 16), dev)
    if codec in (W4_LUT16S, W4_LUT16S_PERM, W4_LUT16S_IL):
        _need(codebook, "codebook", _U16, (16,), dev)
    if codec == W4_SIGNMAG8:
        _need(codebook, "codebook", _U16, (n, k // g, 8), dev)


def w4_quantize_pack(w, codec=W4_DYADIC, *, scales=None, codebook=None, packed=None,
                     stream=None):
    """Quantize a bf16 weight [n, k] and pack two 4-bit indices per byte.

    DYADIC writes ``scales`` (allocated if None); LUT16 reads ``scales`` and
    ``codebook``; SIGNMAG8 reads ``codebook``.  Returns (packed, scales)."""
    _need(w, "w", _U16)
    n, k = w.shape
    if packed is None:
        packed = torch.empty((n, k // 2), dtype=torch.uint8, device=w.device)
    _need(packed, "packed", (torch.uint8,), (n, k // 2))
    if codec == W4_DYADIC and scales is None:
        scales = torch.empty((n, k // 64), dtype=torch.bfloat16, device=w.device)
    _side_tables(codec, n, k, scales, codebook)
    _check(_lib.w4_quantize_pack(codec, n, k, _ptr(w), _ptr(packed), _ptr(scales),
                                 _ptr(codebook), _stream(stream)))
    return packed, scales


def w4_unpack_dequant(packed, codec=W4_DYADIC, *, scales=None, codebook=None, out=None,
                      stream=None):
    """Dense rebuilt weight: bf16 [n, k] (DYADIC, LUT16, LUT16S and its
    variants, DYADIC5) or fp16 (SIGNMAG8)."""
    _need(packed, "packed", (torch.uint8,))
    n, k = packed.shape[0], _k_of(codec, packed)
    _side_tables(codec, n, k, scales, codebook)
    dt = torch.float16 if codec == W4_SIGNMAG8 else torch.bfloat16
    if out is None:
        out = torch.empty((n, k), dtype=dt, device=packed.device)
    _need(out, "out", _U16, (n, k))
    _check(_lib.w4_unpack_dequant(codec, n, k, _ptr(packed), _ptr(scales), _ptr(codebook),
                                  _ptr(out), _stream(stream)))
    return out


def w4_quantize_dyadic5(w, widths=None, *, packed=None, msb=None, scales=None, stream=None):
    """Quantize a bf16 weight [n, k] to W4_DYADIC5 with a width of 3, 4 or 5
    bits per group of 64 (``widths`` uint8 [n, k/64]; None: 5 everywhere).
    Returns (packed [n, k/2], msb [n, k/8], scales [n, k/64]); the matrix calls
    take the high-bit plane ``msb`` as their ``codebook``."""
    _need(w, "w", _U16)
    n, k = w.shape
    if widths is not None:
        _need(widths, "widths", (torch.uint8,), (n, k // 64))
    if packed is None:
        packed = torch.empty((n, k // 2), dtype=torch.uint8, device=w.device)
    if msb is None:
        msb = torch.empty((n, k // 8), dtype=torch.uint8, device=w.device)
    if scales is None:
        scales = torch.empty((n, k // 64), dtype=torch.bfloat16, device=w.device)
    _need(packed, "packed", (torch.uint8,), (n, k // 2))
    _need(msb, "msb", (torch.uint8,), (n, k // 8))
    _need(scales, "scales", _U16, (n, k // 64))
    _check(_lib.w4_quantize_dyadic5(n, k, _ptr(w), _ptr(widths), _ptr(packed), _ptr(msb),
                                    _ptr(scales), _stream(stream)))
    return packed, msb, scales


def w4_lut16_fit(w, iters=25, *, scales=None, codebook=None, stream=None):
    """Fit the LUT16 codec's per-group scale and 16 levels to a bf16 weight
    [n, k] on the GPU (1D k-means per group of 64).  Returns (scales bf16
    [n, k/64], codebook bf16 [n, k/64, 16]), the inputs w4_quantize_pack
    takes for W4_LUT16."""
    _need(w, "w", _U16)
    n, k = w.shape
    if scales is None:
        scales = torch.empty((n, k // 64), dtype=torch.bfloat16, device=w.device)
    if codebook is None:
        codebook = torch.empty((n, k // 64, 16), dtype=torch.bfloat16, device=w.device)
    _need(scales, "scales", _U16, (n, k // 64))
    _need(codebook, "codebook", _U16, (n, k // 64, 16))
    _check(_lib.w4_lut16_fit(n, k, _ptr(w), _ptr(scales), _ptr(codebook), iters,
                             _stream(stream)))
    return scales, codebook


def w4_signmag8_fit(w, iters=25, *, codebook=None, stream=None):
    """Fit the SIGNMAG8 codec's 8 fp16 magnitudes per group of 32 to a bf16
    weight [n, k] on the GPU (1D k-means on |w|).  Returns the codebook
    (float16 [n, k/32, 8]) that w4_quantize_pack takes for W4_SIGNMAG8."""
    _need(w, "w", _U16)
    n, k = w.shape
    if codebook is None:
        codebook = torch.empty((n, k // 32, 8), dtype=torch.float16, device=w.device)
    _need(codebook, "codebook", _U16, (n, k // 32, 8))
    _check(_lib.w4_signmag8_fit(n, k, _ptr(w), _ptr(codebook), iters, _stream(stream)))
    return codebook


def w4_signmag8_fit_warm(w, iters=25, *, codebook=None, params=None, stream=None):
    """Warm-start fit of the SIGNMAG8 magnitudes (the best of 112 parametric
    transforms per group of 32, then Lloyd rounds) on the GPU.  Returns
    (codebook float16 [n, k/32, 8], parameter codes uint8 [n, k/32])."""
    _need(w, "w", _U16)
    n, k = w.shape
    if codebook is None:
        codebook = torch.empty((n, k // 32, 8), dtype=torch.float16, device=w.device)
    if params is None:
        params = torch.empty((n, k // 32), dtype=torch.uint8, device=w.device)
    _need(codebook, "codebook", _U16, (n, k // 32, 8))
    _need(params, "params", (torch.uint8,), (n, k // 32))
    _check(_lib.w4_signmag8_fit_warm(n, k, _ptr(w), _ptr(codebook), _ptr(params), iters,
                                     _stream(stream)))
    return codebook, params


def _matmul(fn, packed, x, codec, scales, codebook, y, y_dtype, stream):
    _need(packed, "packed", (torch.uint8,))
    dev = packed.get_device()  # the current device, as just checked
    n = packed.shape[0]
    k = _k_of(codec, packed)
    _side_tables(codec, n, k, scales, codebook, dev)
    _need(x, "x", _U16, None, dev)
    if x.dim() != 2 or x.shape[1] != k:
        raise ValueError(f"x must be [m, {k}]")
    m = x.shape[0]
    code = W4_BF16 if y_dtype == torch.bfloat16 else W4_F32
    if y is None:
        y = torch.empty((m, n), dtype=torch.bfloat16 if code == W4_BF16 else torch.float32,
                        device=packed.device)
    _need(y, "y", (torch.float32,) if code == W4_F32 else _U16, (m, n), dev)
    _check(fn(codec, n, k, _ptr(packed), _ptr(scales), _ptr(codebook), _ptr(x), m, _ptr(y),
              code, _stream(stream, dev)))
    return y


def w4_lut16s_interleave(packed, scales, out=None, stream=None):
    """The W4_LUT16S_IL records of a LUT16S weight (packed [n, k/2], scales
    [n, k/64], k a multiple of 256) -> uint8 [n, k/256 * 144]."""
    _need(packed, "packed", (torch.uint8,))
    n, k = packed.shape[0], 2 * packed.shape[1]
    _need(scales, "scales", _U16, (n, k // 64))
    if out is None:
        out = torch.empty((n, k // 256 * IL_RECORD), dtype=torch.uint8, device=packed.device)
    _need(out, "out", (torch.uint8,), (n, k // 256 * IL_RECORD))
    _check(_lib.w4_lut16s_interleave(n, k, _ptr(packed), _ptr(scales), _ptr(out),
                                     _stream(stream)))
    return out


def w4_gemv(packed, x, codec=W4_DYADIC, *, scales=None, codebook=None, y=None,
            y_dtype=torch.float32, stream=None):
    """y[m, n] = x[m, k] @ w_hat[n, k]^T for 1 <= m <= 16 (fused dequant)."""
    return _matmul(_lib.w4_gemv, packed, x, codec, scales, codebook, y, y_dtype, stream)


def w4_gemm(packed, x, codec=W4_DYADIC, *, scales=None, codebook=None, y=None,
            y_dtype=torch.float32, stream=None):
    """Y[m, n] = X[m, k] @ w_hat[n, k]^T, bf16 MFMA (fused dequant), any m >= 1."""
    return _matmul(_lib.w4_gemm, packed, x, codec, scales, codebook, y, y_dtype, stream)


def w4_gemm_noalloc(packed, x, codec=W4_DYADIC, *, scales=None, codebook=None, y=None,
                    y_dtype=torch.float32, stream=None):
    """w4_gemm with the library's fixed scratch array instead of an allocated
    workspace (the call itself allocates nothing; pass ``y`` to allocate
    nothing here either).  Overlapping calls on one GPU race."""
    return _matmul(_lib.w4_gemm_noalloc, packed, x, codec, scales, codebook, y, y_dtype, stream)


def w4_linear(packed, x, codec=W4_DYADIC, *, scales=None, codebook=None, y=None,
              y_dtype=torch.float32, stream=None):
    """Y[m, n] = X[m, k] @ w_hat[n, k]^T with the kernel chosen by m (GEMV for
    m <= 16, GEMM above)."""
    return _matmul(_lib.w4_linear, packed, x, codec, scales, codebook, y, y_dtype, stream)


class W4GemvBatch:
    """A planned batch of independent GEMVs (``w4_gemv_batched_plan``), with
    its descriptor table already in device memory.  Call it to launch."""

    def __init__(self, codec, m, y_dtype, table_dev, info, keepalive):
        self.codec, self.m, self.y_dtype = codec, m, y_dtype
        self.table, self.info = table_dev, info
        self._keep = keepalive

    @property
    def total_tiles(self):
        return self.info.total_tiles

    def __call__(self, stream=None):
        _check(_lib.w4_gemv_batched(self.codec, self.m, self.y_dtype, self.table.data_ptr(),
                                    ctypes.byref(self.info), _stream(stream)))


def w4_gemv_batched_plan(problems, codec=W4_DYADIC, y_dtype=torch.float32):
    """problems: list of dicts with packed, x, y and scales / codebook as the
    codec needs.  Validates all of them, uploads the descriptor table and
    returns a W4GemvBatch."""
    code = W4_BF16 if y_dtype == torch.bfloat16 else W4_F32
    arr = (W4Problem * len(problems))()
    m = None
    keep = []
    for i, p in enumerate(problems):
        packed, x, y = p["packed"], p["x"], p["y"]
        _need(packed, "packed", (torch.uint8,))
        n, k = packed.shape[0], _k_of(codec, packed)
        _side_tables(codec, n, k, p.get("scales"), p.get("codebook"))
        _need(x, "x", _U16, (x.shape[0], k))
        _need(y, "y", (torch.float32,) if code == W4_F32 else _U16, (x.shape[0], n))
        if m is None:
            m = x.shape[0]
        elif x.shape[0] != m:
            raise ValueError("all problems of a batch share m")
        arr[i] = W4Problem(packed.data_ptr(), _ptr(p.get("scales")), _ptr(p.get("codebook")),
                           x.data_ptr(), y.data_ptr(), n, k, 0)
        keep.append(p)
    info = W4BatchInfo()
    _check(_lib.w4_gemv_batched_plan(codec, m or 1, code, arr, len(problems),
                                     ctypes.byref(info)))
    dev = problems[0]["packed"].device if problems else torch.device("cuda")
    table = torch.frombuffer(bytearray(bytes(arr)), dtype=torch.uint8).to(dev)
    return W4GemvBatch(codec, m or 1, code, table, info, keep)
