"""Python binding of the MI355X MLA decode library (argument marshalling only).

Every step of the computation runs in the HIP kernels of
``csrc/mla_decode.hip`` behind the C ABI declared in ``include/mla_decode.h``;
this module only checks tensor placement, picks the format codes from tensor
dtypes, passes raw pointers and the current HIP stream through ctypes, and
allocates outputs/workspaces with torch.  There is no fallback: if the shared
library is missing the calls raise.

Tensor conventions:
  bf16 data          torch.bfloat16
  fp8 e4m3fn data    torch.float8_e4m3fn (one fp32 per-tensor scale, a 1-element
                     float32 tensor on the device)
  mxfp4 data         torch.uint8 packed [..., 288] + torch.uint8 e8m0 scales [..., 18]
  split cache        an mxfp4 key cache plus a float8_e4m3fn value cache on the same
                     rows (decode_mixed)
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

from . import build as _build

__all__ = [
    "BF16", "FP8", "MXFP4", "HEADS", "D_QK", "D_V",
    "load", "decode", "workspace_bytes", "choose_num_splits", "recommend_page_size",
    "quantize_fp8", "quantize_mxfp4", "validate", "status_string", "StatusError",
    "mxfp4_scale_buffer", "MIXED", "decode_mixed", "validate_mixed", "new_workspace", "decode_noalloc",
    "NOALLOC_SCRATCH_BYTES", "Q_BF16_FP8_STATIC", "Q_BF16_MXFP4",
]

BF16, FP8, MXFP4 = 0, 1, 2
MIXED = 3  # split cache: mxfp4 K + fp8 V (format code for choose_num_splits)
Q_BF16_FP8_STATIC = 4  # bf16 Q quantised to fp8 inside the decode with a static scale
Q_BF16_MXFP4 = 5  # bf16 Q quantised to mxfp4 inside the decode
HEADS, D_QK, D_V = 16, 576, 512
MXFP4_ROW_BYTES, MXFP4_ROW_SCALES = 288, 18
MAX_SPLITS = 256

_lock = threading.Lock()
_lib = None

_c_int32, _c_int64, _c_size, _c_void = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p
_DECODE_ARGS = [_c_void, _c_int32, _c_void, _c_void, _c_int32, _c_void, _c_int64, _c_void, _c_int32,
                _c_void, _c_void, _c_int32, _c_int32, _c_void, _c_void, _c_size]

EXPORTS = ("mla_decode", "mla_validate", "mla_workspace_bytes", "mla_choose_num_splits",
           "mla_recommend_page_size", "mla_quantize_fp8", "mla_quantize_mxfp4", "mla_stream_read",
           "mla_plan_worklist", "mla_worklist_workspace_bytes", "mla_decode_worklist", "mla_decode_rows",
           "mla_workspace_bytes_rows", "mla_decode_mixed", "mla_validate_mixed", "mla_check_tables",
           "mla_decode_noalloc", "mla_status_string", "mla_abi_version")


class StatusError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status} ({status_string(status)})")
        self.status = status


def load():
    """Load (without building) the in-tree shared library."""
    global _lib
    with _lock:
        if _lib is None:
            path = _build.LIB_PATH
            if not os.path.exists(path):
                raise RuntimeError(f"{path} is missing: run __graft_entry__.build() (or "
                                   f"python -m mla_latent_kv_13_amd.build) first")
            L = ctypes.CDLL(path)
            L.mla_decode.restype = ctypes.c_int
            L.mla_decode.argtypes = _DECODE_ARGS + [_c_void]
            L.mla_validate.restype = ctypes.c_int
            L.mla_validate.argtypes = _DECODE_ARGS
            L.mla_decode_noalloc.restype = ctypes.c_int
            L.mla_decode_noalloc.argtypes = _DECODE_ARGS[:14] + [_c_void]
            L.mla_workspace_bytes.restype = _c_size
            L.mla_workspace_bytes.argtypes = [_c_int32, _c_int32]
            L.mla_choose_num_splits.restype = _c_int32
            L.mla_choose_num_splits.argtypes = [_c_int32, _c_int32, _c_int32, _c_int32, _c_int32]
            L.mla_recommend_page_size.restype = _c_int32
            L.mla_recommend_page_size.argtypes = [_c_int32, _c_int32, _c_int32, _c_int32, _c_int32]
            L.mla_quantize_fp8.restype = ctypes.c_int
            L.mla_quantize_fp8.argtypes = [_c_void, _c_int64, _c_void, _c_void, _c_int32, _c_void]
            L.mla_quantize_mxfp4.restype = ctypes.c_int
            L.mla_quantize_mxfp4.argtypes = [_c_void, _c_int64, _c_int64, _c_void, _c_void, _c_void]
            L.mla_check_tables.restype = ctypes.c_int
            L.mla_check_tables.argtypes = [_c_void, _c_int32, _c_void, ctypes.c_int64, _c_void, _c_int32,
                                           ctypes.c_int64, _c_void]
            L.mla_plan_worklist.restype = ctypes.c_int
            L.mla_plan_worklist.argtypes = [_c_void, _c_int32, _c_int32, _c_int32, _c_void, _c_void, _c_void, _c_void]
            L.mla_worklist_workspace_bytes.restype = _c_size
            L.mla_worklist_workspace_bytes.argtypes = [_c_int32, _c_int32]
            _rows_args = _DECODE_ARGS[:3] + [_c_int32] + _DECODE_ARGS[3:12]
            L.mla_decode_worklist.restype = ctypes.c_int
            L.mla_decode_worklist.argtypes = (_rows_args + [_c_void, _c_int32, _c_void, _c_int32]
                                              + [_c_void, _c_void, _c_size, _c_void])
            L.mla_decode_rows.restype = ctypes.c_int
            L.mla_decode_rows.argtypes = _rows_args + [_c_int32, _c_void, _c_void, _c_size, _c_void]
            L.mla_workspace_bytes_rows.restype = _c_size
            L.mla_workspace_bytes_rows.argtypes = [_c_int32, _c_int32, _c_int32]
            _mixed_args = [_c_void, _c_int32, _c_void, _c_int32, _c_void, _c_void, _c_void, _c_void, _c_int64,
                           _c_void, _c_int32, _c_void, _c_void, _c_int32, _c_int32, _c_void, _c_void, _c_size]
            L.mla_decode_mixed.restype = ctypes.c_int
            L.mla_decode_mixed.argtypes = _mixed_args + [_c_void]
            L.mla_validate_mixed.restype = ctypes.c_int
            L.mla_validate_mixed.argtypes = _mixed_args
            L.mla_stream_read.restype = ctypes.c_int
            L.mla_stream_read.argtypes = [_c_void, _c_int64, _c_void, _c_void]
            L.mla_status_string.restype = ctypes.c_char_p
            L.mla_status_string.argtypes = [ctypes.c_int]
            L.mla_abi_version.restype = _c_int32
            L.mla_abi_version.argtypes = []
            _lib = L
    return _lib


def status_string(status: int) -> str:
    return load().mla_status_string(int(status)).decode()


def _stream(stream=None) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def _fmt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float8_e4m3fn:
        return FP8
    if t.dtype == torch.uint8:
        return MXFP4
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _dev(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("all tensors must be on the GPU")
            if not t.is_contiguous():
                raise ValueError("all tensors must be contiguous")


def workspace_bytes(batch: int, num_splits: int, q_rows: int = HEADS) -> int:
    return int(load().mla_workspace_bytes_rows(int(batch), int(q_rows), int(num_splits)))


def new_workspace(nbytes: int, device) -> torch.Tensor | None:
    """A workspace of nbytes on `device` (None for 0 bytes)."""
    if nbytes <= 0:
        return None
    return torch.empty(int(nbytes), dtype=torch.uint8, device=device)


def choose_num_splits(batch: int, kv_len: int, kv_dtype: int, num_cus: int = 0, *, q_dtype: int = BF16) -> int:
    """Split count for batch requests of about kv_len tokens (mla_choose_num_splits)."""
    return int(load().mla_choose_num_splits(int(batch), int(kv_len), int(q_dtype), int(kv_dtype), int(num_cus)))


def recommend_page_size(batch: int, kv_len: int, q_dtype: int = BF16, kv_dtype: int = FP8, num_cus: int = 0) -> int:
    """Page size for a cache of such requests (mla_recommend_page_size)."""
    return int(load().mla_recommend_page_size(int(batch), int(kv_len), int(q_dtype), int(kv_dtype), int(num_cus)))


def _check_operands(q, kv_cache, kv_scale, out, batch: int, rows: int, what: str = "kv_cache") -> None:
    """Shape and dtype checks the C ABI cannot make from raw pointers (it
    would read or write past a wrong-sized buffer): Q rows, cache row width,
    the padded mxfp4 scale allocation, and the output tensor."""
    fmt = _fmt(kv_cache)
    width = MXFP4_ROW_BYTES if fmt == MXFP4 else D_QK
    if kv_cache.dim() != 2 or kv_cache.shape[1] != width:
        raise ValueError(f"{what} must be [rows, {width}] for its format, got {tuple(kv_cache.shape)}")
    if q.dim() != 3 or q.shape[0] != batch or q.shape[2] != (MXFP4_ROW_BYTES if _fmt(q) == MXFP4 else D_QK):
        raise ValueError(f"q must be [batch, rows, 576] (mxfp4: [batch, rows, 288]), got {tuple(q.shape)}")
    if fmt == MXFP4 and kv_scale is not None:
        need = (MXFP4_ROW_SCALES * kv_cache.shape[0] + 15) // 16 * 16
        have = kv_scale.untyped_storage().nbytes() - kv_scale.storage_offset() * kv_scale.element_size()
        if kv_scale.dtype != torch.uint8 or kv_scale.numel() < MXFP4_ROW_SCALES * kv_cache.shape[0] or have < need:
            raise ValueError(f"mxfp4 scales need {MXFP4_ROW_SCALES} uint8 per row in an allocation of at least "
                             f"{need} bytes (mxfp4_scale_buffer)")
    if fmt == FP8 and kv_scale is not None and (kv_scale.dtype != torch.float32 or kv_scale.numel() < 1):
        raise ValueError("the fp8 cache scale is a 1-element float32 tensor")
    if out is not None and (out.dtype != torch.bfloat16 or tuple(out.shape) != (batch, rows, D_V)):
        raise ValueError(f"out must be bfloat16 [{batch}, {rows}, {D_V}], got {out.dtype} {tuple(out.shape)}")


def _decode_args(q, kv_cache, kv_indptr, page_table, page_size, num_splits, q_scale, kv_scale,
                 page_indptr, out, workspace, q_dtype=None):
    batch = kv_indptr.numel() - 1
    num_rows = kv_cache.shape[0] if kv_cache.dim() else 0
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return [_ptr(q), _fmt(q) if q_dtype is None else int(q_dtype), _ptr(q_scale), _ptr(kv_cache), _fmt(kv_cache), _ptr(kv_scale), num_rows,
            _ptr(kv_indptr), batch, _ptr(page_table), _ptr(page_indptr), int(page_size), int(num_splits),
            _ptr(out), _ptr(workspace), ws_bytes]


def validate(q, kv_cache, kv_indptr, page_table, page_size, num_splits, *, q_scale=None, kv_scale=None,
             page_indptr=None, out=None, workspace=None) -> int:
    """Host-side argument check (no GPU work); returns the status code."""
    return int(load().mla_validate(*_decode_args(q, kv_cache, kv_indptr, page_table, page_size, num_splits,
                                                 q_scale, kv_scale, page_indptr, out, workspace)))


def decode(q: torch.Tensor, kv_cache: torch.Tensor, kv_indptr: torch.Tensor, page_table: torch.Tensor,
           page_size: int, num_splits: int | None = None, *, q_scale=None, kv_scale=None,
           page_indptr=None, out=None, workspace=None, kv_len_hint: int | None = None, stream=None,
           q_fp8_scale=None, q_to_mxfp4: bool = False):
    """MLA decode; returns out [batch,R,512] bf16 (enqueued on the current stream).

    q          [B,R,576] bf16 / float8_e4m3fn, or [B,R,288] uint8 (mxfp4, with q_scale e8m0 [B*R,18]);
               R = q_seq_len x heads query rows per request (16 for single-token decode)
    kv_cache   [R,576] bf16 / float8_e4m3fn, or [R,288] uint8 (mxfp4, with kv_scale e8m0 [R,18])
    kv_indptr  int32 [B+1] token offsets; page_table int32 page ids; page_indptr optional int32 [B]
    q_fp8_scale  with bf16 q over the fp8 cache: a 1-element float32 static scale; the decode then
               quantises q to fp8 itself, code for code as quantize_fp8(q, q_fp8_scale)
               (MLA_Q_BF16_FP8_STATIC), in place of a separate quantiser launch
    q_to_mxfp4 with bf16 q over the mxfp4 cache: the decode quantises q to mxfp4 itself, code for
               code and scale for scale as quantize_mxfp4 (MLA_Q_BF16_MXFP4)
    """
    batch = kv_indptr.numel() - 1
    rows = _q_rows(q, batch)
    _check_operands(q, kv_cache, kv_scale, out, batch, rows)
    q_dtype = _fmt(q)
    if q_fp8_scale is not None:
        if q.dtype != torch.bfloat16 or _fmt(kv_cache) != FP8 or q_scale is not None:
            raise ValueError("q_fp8_scale takes bf16 q over the fp8 cache, without q_scale")
        if q_fp8_scale.dtype != torch.float32 or q_fp8_scale.numel() < 1:
            raise ValueError("q_fp8_scale is a 1-element float32 tensor")
        q_scale, q_dtype = q_fp8_scale, Q_BF16_FP8_STATIC
    if q_to_mxfp4:
        if q.dtype != torch.bfloat16 or _fmt(kv_cache) != MXFP4 or q_scale is not None:
            raise ValueError("q_to_mxfp4 takes bf16 q over the mxfp4 cache, without q_scale")
        q_dtype = Q_BF16_MXFP4
    if num_splits is None:
        # one workgroup per 16-row query group: the occupancy is batch x groups
        hint = kv_len_hint if kv_len_hint is not None else max(1, kv_cache.shape[0] // max(batch, 1))
        num_splits = choose_num_splits(batch * (rows // HEADS), hint, _fmt(kv_cache), q_dtype=q_dtype)
    if out is None:
        out = torch.empty((batch, rows, D_V), dtype=torch.bfloat16, device=kv_cache.device)
    if workspace is None and batch > 0:
        workspace = new_workspace(workspace_bytes(batch, num_splits, rows), kv_cache.device)
    _dev(q, kv_cache, kv_indptr, page_table, q_scale, kv_scale, page_indptr, out, workspace)
    args = _decode_args(q, kv_cache, kv_indptr, page_table, page_size, num_splits, q_scale, kv_scale, page_indptr,
                        out, workspace, q_dtype)
    L = _lib or load()
    if rows == HEADS:
        rc = L.mla_decode(*args, _stream(stream))
    else:
        rc = L.mla_decode_rows(*args[:3], rows, *args[3:], _stream(stream))
    if rc:
        raise StatusError("mla_decode" if rows == HEADS else "mla_decode_rows", rc)
    return out


NOALLOC_SCRATCH_BYTES = 32 << 20


def decode_noalloc(q: torch.Tensor, kv_cache: torch.Tensor, kv_indptr: torch.Tensor, page_table: torch.Tensor,
                   page_size: int, num_splits: int, out: torch.Tensor, *, q_scale=None, kv_scale=None,
                   page_indptr=None, stream=None):
    """mla_decode_noalloc: single-token decode into a caller-allocated `out`
    [batch,16,512] bf16 with the split partials in the library's static
    per-GPU scratch (workspace_bytes(batch, num_splits) must not exceed
    NOALLOC_SCRATCH_BYTES).  Nothing is allocated; calls that overlap on one
    GPU race on the scratch."""
    batch = kv_indptr.numel() - 1
    rows = _q_rows(q, batch)
    if rows != HEADS:
        raise ValueError("decode_noalloc takes 16 query rows per request")
    if out is None:
        raise ValueError("decode_noalloc writes into a caller-allocated out")
    _check_operands(q, kv_cache, kv_scale, out, batch, rows)
    _dev(q, kv_cache, kv_indptr, page_table, q_scale, kv_scale, page_indptr, out)
    args = _decode_args(q, kv_cache, kv_indptr, page_table, page_size, num_splits, q_scale, kv_scale, page_indptr,
                        out, None)
    rc = (_lib or load()).mla_decode_noalloc(*args[:14], _stream(stream))
    if rc:
        raise StatusError("mla_decode_noalloc", rc)
    return out


def _mixed_args(q, k_cache, k_scale, v_cache, v_scale, kv_indptr, page_table, page_size, num_splits, q_scale,
                page_indptr, out, workspace):
    batch = kv_indptr.numel() - 1
    rows = _q_rows(q, batch)
    num_rows = k_cache.shape[0] if k_cache.dim() else 0
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return [_ptr(q), _fmt(q), _ptr(q_scale), rows, _ptr(k_cache), _ptr(k_scale), _ptr(v_cache), _ptr(v_scale),
            num_rows, _ptr(kv_indptr), batch, _ptr(page_table), _ptr(page_indptr), int(page_size), int(num_splits),
            _ptr(out), _ptr(workspace), ws_bytes]


def validate_mixed(q, k_cache, k_scale, v_cache, v_scale, kv_indptr, page_table, page_size, num_splits, *,
                   q_scale=None, page_indptr=None, out=None, workspace=None) -> int:
    """Host-side argument check of decode_mixed (no GPU work); returns the status code."""
    return int(load().mla_validate_mixed(*_mixed_args(q, k_cache, k_scale, v_cache, v_scale, kv_indptr, page_table,
                                                      page_size, num_splits, q_scale, page_indptr, out, workspace)))


def decode_mixed(q: torch.Tensor, k_cache: torch.Tensor, k_scale: torch.Tensor, v_cache: torch.Tensor,
                 v_scale: torch.Tensor, kv_indptr: torch.Tensor, page_table: torch.Tensor, page_size: int,
                 num_splits: int | None = None, *, q_scale=None, page_indptr=None, out=None, workspace=None,
                 kv_len_hint: int | None = None, stream=None):
    """MLA decode over a split cache (mla_decode_mixed): logits from the mxfp4
    keys, outputs from the fp8 values of the same rows.

    q        [B,R,576] bf16, or [B,R,288] uint8 mxfp4 with q_scale e8m0 [B*R,18]
    k_cache  [rows,288] uint8 packed e2m1, k_scale e8m0 [rows,18] (mxfp4_scale_buffer)
    v_cache  [rows,576] float8_e4m3fn, v_scale 1-element float32 (only dims 0..511 are read)
    Returns out [B,R,512] bf16 (enqueued on the current stream).
    """
    batch = kv_indptr.numel() - 1
    rows = _q_rows(q, batch)
    _check_operands(q, k_cache, k_scale, out, batch, rows, "k_cache")
    if v_cache.dim() != 2 or v_cache.shape[1] != D_QK:
        raise ValueError(f"v_cache must be [rows, {D_QK}], got {tuple(v_cache.shape)}")
    if num_splits is None:
        hint = kv_len_hint if kv_len_hint is not None else max(1, k_cache.shape[0] // max(batch, 1))
        num_splits = choose_num_splits(batch * (rows // HEADS), hint, MIXED, q_dtype=_fmt(q))
    if out is None:
        out = torch.empty((batch, rows, D_V), dtype=torch.bfloat16, device=k_cache.device)
    if workspace is None and batch > 0:
        workspace = new_workspace(workspace_bytes(batch, num_splits, rows), k_cache.device)
    _dev(q, k_cache, k_scale, v_cache, v_scale, kv_indptr, page_table, q_scale, page_indptr, out, workspace)
    if k_cache.dtype != torch.uint8 or v_cache.dtype != torch.float8_e4m3fn:
        raise TypeError("decode_mixed takes a uint8 mxfp4 key cache and a float8_e4m3fn value cache")
    if v_cache.shape[0] != k_cache.shape[0]:
        raise ValueError("the key and value caches must hold the same rows")
    args = _mixed_args(q, k_cache, k_scale, v_cache, v_scale, kv_indptr, page_table, page_size, num_splits, q_scale,
                       page_indptr, out, workspace)
    rc = (_lib or load()).mla_decode_mixed(*args, _stream(stream))
    if rc:
        raise StatusError("mla_decode_mixed", rc)
    return out


def _q_rows(q, batch: int) -> int:
    """Query rows per request from Q's element count (576 values, or 288 packed
    bytes, per row)."""
    if batch <= 0:
        return HEADS
    per_row = 288 if q.dtype == torch.uint8 else 576
    n = q.numel() // per_row
    if n % batch:
        raise ValueError("q does not hold a whole number of rows per request")
    return n // batch


def quantize_fp8(x: torch.Tensor, scale: torch.Tensor | float | None = None, stream=None, out=None):
    """Per-tensor OCP e4m3fn quantisation of a bf16 tensor on the device.

    scale None -> dynamic (max|x| / 448, computed on the device); a float or a
    1-element float32 device tensor -> static.  out: optional preallocated
    float8_e4m3fn tensor of x's shape.  Returns (codes, scale_tensor).
    """
    _dev(x)
    if x.dtype != torch.bfloat16:
        raise TypeError("quantize_fp8 expects bfloat16 input")
    dynamic = scale is None
    if dynamic:
        sc = torch.empty(1, dtype=torch.float32, device=x.device)
    elif isinstance(scale, torch.Tensor):
        sc = scale.to(device=x.device, dtype=torch.float32).reshape(1).contiguous()
    else:
        sc = torch.tensor([float(scale)], dtype=torch.float32, device=x.device)
    codes = torch.empty(x.shape, dtype=torch.float8_e4m3fn, device=x.device) if out is None else out
    if codes.shape != x.shape or codes.dtype != torch.float8_e4m3fn:
        raise ValueError("out must be a float8_e4m3fn tensor of the input's shape")
    _dev(codes)
    rc = load().mla_quantize_fp8(x.data_ptr(), x.numel(), codes.data_ptr(), sc.data_ptr(), int(dynamic),
                                 _stream(stream))
    if rc:
        raise StatusError("mla_quantize_fp8", rc)
    return codes, sc


def mxfp4_scale_buffer(rows: int, device) -> torch.Tensor:
    """An e8m0 scale array [rows, 18] whose allocation is padded to 16 bytes."""
    n = rows * MXFP4_ROW_SCALES
    base = torch.empty(((n + 15) // 16) * 16, dtype=torch.uint8, device=device)
    return base[:n].view(rows, MXFP4_ROW_SCALES)


def quantize_mxfp4(x: torch.Tensor, stream=None, out=None):
    """OCP MX mxfp4 quantisation of a bf16 tensor [..., cols] (cols % 32 == 0).

    Returns (packed uint8 [..., cols/2], e8m0 uint8 [..., cols/32]); for 576-wide
    rows the scale array's allocation is padded as mla_decode requires.  out:
    optional preallocated (packed, scales) pair of those shapes.
    """
    _dev(x)
    if x.dtype != torch.bfloat16:
        raise TypeError("quantize_mxfp4 expects bfloat16 input")
    cols = x.shape[-1]
    rows = x.numel() // cols if cols else 0
    if out is None:
        packed = torch.empty(x.shape[:-1] + (cols // 2,), dtype=torch.uint8, device=x.device)
        nsc = rows * (cols // 32)
        base = torch.empty(max(16, ((nsc + 15) // 16) * 16), dtype=torch.uint8, device=x.device)
        scales = base[:nsc].view(x.shape[:-1] + (cols // 32,))
    else:
        packed, scales = out
        if (packed.shape != x.shape[:-1] + (cols // 2,) or scales.shape != x.shape[:-1] + (cols // 32,)
                or packed.dtype != torch.uint8 or scales.dtype != torch.uint8):
            raise ValueError("out must be uint8 (packed [..., cols/2], scales [..., cols/32])")
        _dev(packed, scales)
    rc = load().mla_quantize_mxfp4(x.data_ptr(), rows, cols, packed.data_ptr(), scales.data_ptr(), _stream(stream))
    if rc:
        raise StatusError("mla_quantize_mxfp4", rc)
    return packed, scales


def stream_read(buf: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Enqueue one streaming read of the whole of `buf` (measurement helper;
    `sink` is a 4-byte device tensor that the kernel almost never writes)."""
    _dev(buf)
    _dev(sink)
    if not buf.is_contiguous():
        raise ValueError("stream_read needs a contiguous buffer")
    nbytes = buf.numel() * buf.element_size()
    rc = load().mla_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), _stream(stream))
    if rc:
        raise StatusError("mla_stream_read", rc)


def plan_worklist(kv_indptr, num_cus: int = 0, max_items: int | None = None):
    """Host work-list plan for a ragged batch (mla_plan_worklist).

    kv_indptr: host int32 token offsets [B+1] (a CPU tensor, numpy array or
    list).  Returns (items int32 [n, 4] CPU tensor {request, first token,
    tokens, slot}, req int32 [B, 2] CPU tensor {first slot, items}, num_slots).
    """
    ind = torch.as_tensor(kv_indptr, dtype=torch.int32).contiguous().cpu()
    batch = ind.numel() - 1
    if max_items is None:
        total = int(ind[-1] - ind[0]) if batch > 0 else 0
        max_items = batch + total // 256 + 1
    items = torch.empty((max(max_items, 1), 4), dtype=torch.int32)
    req = torch.empty((max(batch, 1), 2), dtype=torch.int32)
    n_items, n_slots = ctypes.c_int32(0), ctypes.c_int32(0)
    rc = load().mla_plan_worklist(ind.data_ptr(), batch, int(num_cus), int(max_items), items.data_ptr(),
                                  req.data_ptr(), ctypes.addressof(n_items), ctypes.addressof(n_slots))
    if rc:
        raise StatusError("mla_plan_worklist", rc)
    return items[: n_items.value].clone(), req[:batch].clone(), n_slots.value


def check_tables(kv_indptr, page_table, page_size: int, num_kv_rows: int, page_indptr=None) -> None:
    """Check host copies of the index tables against the cache (mla_check_tables).

    Every token must map to a physical row in [0, num_kv_rows) under the
    paging rule of `decode`.  Tables may be CPU tensors, numpy arrays or
    lists (device tensors are copied to the host).  Raises ValueError naming
    the first bad request, or StatusError for a size or argument error.
    """
    ind = torch.as_tensor(kv_indptr, dtype=torch.int32).detach().contiguous().cpu()
    pt = torch.as_tensor(page_table, dtype=torch.int32).detach().contiguous().cpu().reshape(-1)
    pi = None if page_indptr is None else torch.as_tensor(page_indptr, dtype=torch.int32).detach().contiguous().cpu()
    batch = ind.numel() - 1
    if batch < 0:
        raise ValueError("kv_indptr needs at least one entry")
    if pi is not None and pi.numel() < batch:
        raise ValueError("page_indptr needs one entry per request")
    bad = ctypes.c_int32(-1)
    rc = load().mla_check_tables(ind.data_ptr(), batch, pt.data_ptr() if pt.numel() else None, pt.numel(),
                                 None if pi is None else pi.data_ptr(), int(page_size), int(num_kv_rows),
                                 ctypes.addressof(bad))
    if rc and bad.value >= 0:
        raise ValueError(f"request {bad.value}: offsets decrease or a token maps outside the page table "
                         f"or the {num_kv_rows}-row cache")
    if rc:
        raise StatusError("mla_check_tables", rc)


def worklist_workspace_bytes(num_slots: int, q_rows: int = HEADS) -> int:
    return int(load().mla_worklist_workspace_bytes(int(num_slots), int(q_rows)))


def decode_worklist(q, kv_cache, kv_indptr, page_table, page_size, items, req, num_slots, *, q_scale=None,
                    kv_scale=None, page_indptr=None, out=None, workspace=None, stream=None):
    """MLA decode over a work-list plan (mla_decode_worklist); items / req are
    device copies of plan_worklist's tensors.  Returns out [batch,16,512] bf16."""
    batch = kv_indptr.numel() - 1
    rows = _q_rows(q, batch)
    _check_operands(q, kv_cache, kv_scale, out, batch, rows)
    if out is None:
        out = torch.empty((batch, rows, D_V), dtype=torch.bfloat16, device=kv_cache.device)
    if workspace is None and num_slots > 0:
        workspace = new_workspace(worklist_workspace_bytes(num_slots, rows), kv_cache.device)
    _dev(q, kv_cache, kv_indptr, page_table, q_scale, kv_scale, page_indptr, out, workspace, items, req)
    args = _decode_args(q, kv_cache, kv_indptr, page_table, page_size, 1, q_scale, kv_scale, page_indptr, out,
                        workspace)
    rc = (_lib or load()).mla_decode_worklist(*args[:3], rows, *args[3:12], _ptr(items), items.shape[0], _ptr(req),
                                              int(num_slots), *args[13:], _stream(stream))
    if rc:
        raise StatusError("mla_decode_worklist", rc)
    return out
