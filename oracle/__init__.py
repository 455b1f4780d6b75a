"""Reference oracle for single-token MLA decode (test infrastructure only).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` import this package.  The product library never does, and this
package imports nothing from the product: the two share no code.

The arithmetic lives in ``oracle.c`` (plain fp64 C, see its header for the
passages it follows).  This module only builds/loads that library and marshals
numpy arrays into it.

Parity status of each entry point (pins live in ``tests/test_oracle_*.py``):
  * codecs (bf16, e4m3fn, e2m1, e8m0)       pinned exhaustively
  * fp8 / mxfp4 quantisers                   pinned (library casts, worked cases, bounds)
  * decode (unsplit and split-wise)          pinned (library SDPA, closed forms, invariants)
  * decode over a split cache (mxfp4 K, fp8 V) pinned (library SDPA, one-token and constant-key forms)
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_BUILD = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD, "liboracle.so")
_lock = threading.Lock()
_lib = None

HEADS = 16
D_QK = 576
D_V = 512
PACKED = 288
NBLK = 18

BF16, FP8, MXFP4 = 0, 1, 2
_DTYPES = {"bf16": BF16, "fp8": FP8, "mxfp4": MXFP4}


_CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math", "-ffp-contract=off"]


def build(force: bool = True) -> str:
    """Compile oracle.c into _build/liboracle.so with gcc (OpenMP, no fast-math)."""
    os.makedirs(_BUILD, exist_ok=True)
    src = os.path.join(_HERE, "oracle.c")
    if not force and os.path.exists(_LIB_PATH) and os.path.getmtime(_LIB_PATH) >= os.path.getmtime(src):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp"
    subprocess.run(["gcc", *_CFLAGS, src, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def source() -> str:
    """The text of oracle.c (the mutation tests patch a copy of it)."""
    with open(os.path.join(_HERE, "oracle.c")) as f:
        return f.read()


def build_variant(text: str, path: str, extra_flags=()) -> str:
    """Compile C text (a patched copy of oracle.c) with the oracle's own flags
    into the shared library `path`; test infrastructure for mutation tests and
    sanitizer builds."""
    d = os.path.dirname(os.path.abspath(path))
    os.makedirs(d, exist_ok=True)
    src = os.path.splitext(path)[0] + ".c"
    with open(src, "w") as f:
        f.write(text)
    subprocess.run(["gcc", *_CFLAGS, *extra_flags, src, "-o", path, "-lm"], check=True)
    return path


@contextlib.contextmanager
def variant(path: str):
    """Route every call of this module to the library at `path` (a variant
    built by build_variant) inside the with-block, then restore the oracle."""
    global _lib
    lib()
    with _lock:
        saved = _lib
        _lib = _configure(ctypes.CDLL(path))
    try:
        yield
    finally:
        with _lock:
            _lib = saved


class _Problem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("q_dtype", ctypes.c_int32),
        ("q", ctypes.c_void_p),
        ("q_scale", ctypes.c_double),
        ("q_e8m0", ctypes.c_void_p),
        ("kv_dtype", ctypes.c_int32),
        ("kv", ctypes.c_void_p),
        ("kv_rows", ctypes.c_int64),
        ("kv_scale", ctypes.c_double),
        ("kv_e8m0", ctypes.c_void_p),
        ("kv_indptr", ctypes.c_void_p),
        ("page_indptr", ctypes.c_void_p),
        ("page_table", ctypes.c_void_p),
        ("page_table_len", ctypes.c_int64),
        ("page_size", ctypes.c_int32),
        ("rows", ctypes.c_int32),
        ("v", ctypes.c_void_p),
        ("v_dtype", ctypes.c_int32),
        ("v_scale", ctypes.c_double),
    ]


def _configure(L):
    L.orc_bf16_to_f64.restype = ctypes.c_double
    L.orc_bf16_to_f64.argtypes = [ctypes.c_uint16]
    L.orc_e4m3fn_to_f64.restype = ctypes.c_double
    L.orc_e4m3fn_to_f64.argtypes = [ctypes.c_uint8]
    L.orc_e2m1_to_f64.restype = ctypes.c_double
    L.orc_e2m1_to_f64.argtypes = [ctypes.c_uint8]
    L.orc_e8m0_to_f64.restype = ctypes.c_double
    L.orc_e8m0_to_f64.argtypes = [ctypes.c_uint8]
    L.orc_f64_to_bf16.restype = ctypes.c_uint16
    L.orc_f64_to_bf16.argtypes = [ctypes.c_double]
    L.orc_amax_bf16.restype = ctypes.c_float
    L.orc_amax_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int64]
    L.orc_fp8_scale_from_amax.restype = ctypes.c_float
    L.orc_fp8_scale_from_amax.argtypes = [ctypes.c_float]
    L.orc_quant_fp8.restype = ctypes.c_int
    L.orc_quant_fp8.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p]
    L.orc_quant_mxfp4.restype = ctypes.c_int
    L.orc_quant_mxfp4.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                  ctypes.c_void_p, ctypes.c_void_p]
    L.orc_decode.restype = ctypes.c_int
    L.orc_decode.argtypes = [ctypes.POINTER(_Problem), ctypes.c_int32, ctypes.c_void_p,
                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32]
    return L


def lib():
    global _lib
    with _lock:
        if _lib is None:
            build(force=False)  # compiles only when missing or older than oracle.c
            _lib = _configure(ctypes.CDLL(_LIB_PATH))
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _u16(a) -> np.ndarray:
    """Accept bf16 bits as a numpy uint16/int16 array or a torch bfloat16 tensor."""
    if hasattr(a, "view") and hasattr(a, "dtype") and "bfloat16" in str(a.dtype):
        import torch  # local: only the torch->bits reinterpretation needs it
        return np.ascontiguousarray(a.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16))
    a = np.ascontiguousarray(a)
    if a.dtype == np.int16:
        a = a.view(np.uint16)
    assert a.dtype == np.uint16, a.dtype
    return a


# ------------------------------------------------------------------ codecs

def bf16_to_f64(bits) -> np.ndarray:
    b = _u16(bits)
    f = lib().orc_bf16_to_f64
    return np.vectorize(f, otypes=[np.float64])(b) if b.size else np.zeros(b.shape)


def e4m3fn_to_f64(codes) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    return np.vectorize(lib().orc_e4m3fn_to_f64, otypes=[np.float64])(c)


def e2m1_to_f64(nibbles) -> np.ndarray:
    c = np.ascontiguousarray(nibbles, dtype=np.uint8)
    return np.vectorize(lib().orc_e2m1_to_f64, otypes=[np.float64])(c)


def e8m0_to_f64(codes) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    return np.vectorize(lib().orc_e8m0_to_f64, otypes=[np.float64])(c)


def f64_to_bf16(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    return np.vectorize(lib().orc_f64_to_bf16, otypes=[np.uint16])(x)


# -------------------------------------------------------------- quantisers

def amax_bf16(bits) -> float:
    b = _u16(bits)
    return float(lib().orc_amax_bf16(_ptr(b), b.size))


def fp8_scale_from_amax(amax: float) -> float:
    return float(np.float32(lib().orc_fp8_scale_from_amax(ctypes.c_float(amax))))


def quant_fp8(bits, scale: float | None = None):
    """Per-tensor e4m3fn quantisation. Returns (codes uint8 same shape, fp32 scale)."""
    b = _u16(bits)
    if scale is None:
        scale = fp8_scale_from_amax(amax_bf16(b))
    out = np.empty(b.shape, dtype=np.uint8)
    rc = lib().orc_quant_fp8(_ptr(b), b.size, ctypes.c_float(scale), _ptr(out))
    if rc:
        raise ValueError(f"orc_quant_fp8 failed: {rc}")
    return out, float(np.float32(scale))


def quant_mxfp4(bits):
    """OCP MX mxfp4 over the last axis. Returns (packed [..., n/2] u8, e8m0 [..., n/32] u8)."""
    b = _u16(bits)
    cols = b.shape[-1]
    rows = b.size // cols if cols else 0
    packed = np.empty(b.shape[:-1] + (cols // 2,), dtype=np.uint8)
    scales = np.empty(b.shape[:-1] + (cols // 32,), dtype=np.uint8)
    rc = lib().orc_quant_mxfp4(_ptr(b), rows, cols, _ptr(packed), _ptr(scales))
    if rc:
        raise ValueError(f"orc_quant_mxfp4 failed: {rc}")
    return packed, scales


# ------------------------------------------------------------------ decode

def decode(q, kv, kv_indptr, page_table, page_size, *, q_dtype="bf16", kv_dtype="bf16",
           q_scale=1.0, q_e8m0=None, kv_scale=1.0, kv_e8m0=None, page_indptr=None,
           num_splits=0, pairs=None, nthreads=None, v=None, v_dtype="fp8", v_scale=1.0):
    """fp64 MLA decode.

    q        : bf16 bits [B,rows,576] | e4m3fn codes [B,rows,576] | packed mxfp4 [B,rows,288]
               (rows = q_seq_len x heads query rows per request; 16 for
               single-token decode with 16 heads)
    kv       : physical rows, bf16 bits [R,576] | e4m3fn [R,576] | packed [R,288]
    v        : optional value cache with the same physical rows, bf16 bits or
               e4m3fn codes [R,576] (``v_dtype``, fp8 scale ``v_scale``); V is
               then its dims 0..511 instead of the key rows'
    returns  : (out_f64 [B,rows,512], out_bf16_bits [B,rows,512]); rows of pairs not
               selected (when ``pairs`` is given) are NaN / 0.
    """
    qd, kd = _DTYPES[q_dtype], _DTYPES[kv_dtype]
    qa = _u16(q) if qd == BF16 else np.ascontiguousarray(q, dtype=np.uint8)
    ka = _u16(kv) if kd == BF16 else np.ascontiguousarray(kv, dtype=np.uint8)
    ind = np.ascontiguousarray(kv_indptr, dtype=np.int32)
    pt = np.ascontiguousarray(page_table, dtype=np.int32)
    pind = None if page_indptr is None else np.ascontiguousarray(page_indptr, dtype=np.int32)
    qe = None if q_e8m0 is None else np.ascontiguousarray(q_e8m0, dtype=np.uint8)
    ke = None if kv_e8m0 is None else np.ascontiguousarray(kv_e8m0, dtype=np.uint8)
    B = ind.size - 1
    P = _Problem()
    P.batch = B
    P.q_dtype = qd
    P.q = _ptr(qa)
    P.q_scale = float(q_scale)
    P.q_e8m0 = _ptr(qe)
    P.kv_dtype = kd
    P.kv = _ptr(ka)
    P.kv_rows = ka.shape[0]
    P.kv_scale = float(kv_scale)
    P.kv_e8m0 = _ptr(ke)
    P.kv_indptr = _ptr(ind)
    P.page_indptr = _ptr(pind)
    P.page_table = _ptr(pt)
    P.page_table_len = pt.size
    P.page_size = int(page_size)
    rows = (qa.size // (B * (288 if qd == MXFP4 else 576))) if B > 0 else HEADS
    P.rows = rows
    va = None
    if v is not None:
        vd = _DTYPES[v_dtype]
        if vd == MXFP4:
            raise ValueError("a separate value cache is bf16 or fp8")
        va = _u16(v) if vd == BF16 else np.ascontiguousarray(v, dtype=np.uint8)
        if va.shape[0] != ka.shape[0] or va.size != ka.shape[0] * D_QK:
            raise ValueError("the value cache must hold the key cache's rows, 576 values each")
        P.v = _ptr(va)
        P.v_dtype = vd
        P.v_scale = float(v_scale)
    out = np.full((B, rows, D_V), np.nan, dtype=np.float64)
    outb = np.zeros((B, rows, D_V), dtype=np.uint16)
    sel = None
    if pairs is not None:
        sel = np.ascontiguousarray(np.asarray(pairs, dtype=np.int32).reshape(-1, 2))
    if nthreads is None:
        nthreads = len(os.sched_getaffinity(0))
    rc = lib().orc_decode(ctypes.byref(P), int(num_splits), _ptr(out), _ptr(outb), _ptr(sel),
                          0 if sel is None else sel.shape[0], int(nthreads))
    if rc:
        raise ValueError(f"orc_decode failed: {rc}")
    return out, outb
