"""MXFP4 fake quantization on AMD Instinct MI355X (gfx950).

Thin ctypes binding over libmxfp4.so (include/mxfp4.h): argument marshalling
only -- every step of the method runs in the library's HIP kernels.  torch is
used for device memory and streams.  There is no CPU fallback: if the library
is missing, or a tensor is not on the GPU, the calls raise.

Functions with the C names take torch tensors (or None) for every pointer
argument and enqueue on torch's current stream:

    mxfp4_qdq_fwd(x, axis, y_row, mask_row, scales_row, y_col, mask_col, scales_col,
                  block=32, rule="floor", scale_factor=6.0)
    mxfp4_ste_bwd(grad_out, mask, grad_in, layout, block=32, group_list=None,
                  group_list_type=1)
    mxfp4_quant_pack(x, codes, scales, y=None, mask=None, block=32, rule="floor",
                     scale_factor=6.0)
    mxfp4_grouped_qdq(x, group_list, y, mask=None, scales=None, block=32,
                      rule="floor", scale_factor=6.0, group_list_type=1)
    mxfp4_quant_pack_kmajor(x, codes_t, scales_t, block=32, rule="floor",
                            scale_factor=6.0, group_list=None, group_list_type=1)
    mxfp4_dequant(codes, scales, y, block=32)
    mxfp8_quant(x, q, scales, fmt="e4m3")

Tensor conventions: x / y / grads are bfloat16 or float32, 2-D contiguous
(higher ranks are viewed as rows x last-dim); bitmaps are int32 tensors (the
uint32 bit patterns); scales and codes are uint8; group_list is int64 on the
device, or a CPU tensor / sequence, which is validated (counts >= 0 summing
to rows, or non-decreasing ends ending at rows) and copied to the device.  The alloc_* helpers allocate outputs of the documented shapes.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "ROW", "COL", "GROUPED", "FLOOR", "AMCT",
    "mxfp4_qdq_fwd", "mxfp4_ste_bwd", "mxfp4_quant_pack", "mxfp4_grouped_qdq",
    "mxfp4_quant_pack_kmajor", "mxfp4_dequant", "mxfp8_quant",
    "mxfp4_mask_to_bool", "mxfp4_saturation_mask", "mxfp4_qdq_fwd_rows_batch", "mxfp4_ste_bwd_rows_batch",
    "mxfp4_last_error", "mxfp4_version", "library_path",
    "row_mask_shape", "col_mask_shape", "grouped_mask_rows_max", "grouped_scale_rows_max",
    "kmajor_k_blocks",
]

ROW, COL, GROUPED = 1, 2, 4
FLOOR, AMCT = 0, 1
_F32, _BF16 = 0, 1
_OK, _EINVAL, _EUNSUPPORTED, _EHIP = 0, 1, 2, 3

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.environ.get("MXFP4_LIBRARY") or os.path.join(_HERE, "libmxfp4.so")


class _Desc(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("block", ctypes.c_int32), ("rule", ctypes.c_int32),
                ("reserved0", ctypes.c_int32), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("scale_factor", ctypes.c_float), ("reserved1", ctypes.c_int32)]


class _MxOperand(ctypes.Structure):
    """mxfp4_mx_operand_t (include/mxfp4.h)."""
    _fields_ = [("data", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("fmt", ctypes.c_int32),
                ("block", ctypes.c_int32), ("ld", ctypes.c_int64), ("ld_scales", ctypes.c_int64),
                ("group_stride", ctypes.c_int64), ("group_stride_scales", ctypes.c_int64)]


class _RowItem(ctypes.Structure):
    """mxfp4_row_item_t (include/mxfp4.h)."""
    _fields_ = [("x", ctypes.c_void_p), ("y", ctypes.c_void_p), ("mask", ctypes.c_void_p),
                ("scales", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64)]


class _SteItem(ctypes.Structure):
    """mxfp4_ste_item_t (include/mxfp4.h)."""
    _fields_ = [("grad_out", ctypes.c_void_p), ("mask", ctypes.c_void_p), ("grad_in", ctypes.c_void_p),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64)]


BATCH_MAX = 8
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"libmxfp4.so not found at {_LIB_PATH}; build it with "
                "`python -m mxfp4_fake_quantization_amd.build` (hipcc, gfx950)")
        lib = ctypes.CDLL(_LIB_PATH)
        vp, i32 = ctypes.c_void_p, ctypes.c_int32
        dp = ctypes.POINTER(_Desc)
        lib.mxfp4_qdq_fwd.argtypes = [dp, i32, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.mxfp4_ste_bwd.argtypes = [dp, i32, vp, vp, vp, vp, i32, i32, vp]
        lib.mxfp4_mask_to_bool.argtypes = [i32, ctypes.c_int64, ctypes.c_int64, vp, vp, vp]
        lib.mxfp4_qdq_fwd_rows_batch.argtypes = [dp, i32, ctypes.POINTER(_RowItem), vp]
        lib.mxfp4_ste_bwd_rows_batch.argtypes = [dp, i32, ctypes.POINTER(_SteItem), vp]
        lib.mxfp4_quant_pack.argtypes = [dp, vp, vp, vp, vp, vp, vp]
        lib.mxfp4_grouped_qdq.argtypes = [dp, vp, vp, i32, i32, vp, vp, vp, vp]
        lib.mxfp4_quant_pack_kmajor.argtypes = [dp, vp, vp, i32, i32, ctypes.c_int64, vp, vp, vp]
        lib.mxfp4_dequant.argtypes = [dp, vp, vp, vp, vp]
        lib.mxfp8_quant.argtypes = [dp, i32, vp, vp, vp, vp]
        lib.mxfp8_quant_kmajor.argtypes = [dp, i32, vp, vp, i32, i32, ctypes.c_int64, vp, vp, vp]
        op = ctypes.POINTER(_MxOperand)
        i64 = ctypes.c_int64
        lib.mxfp4_grouped_matmul.argtypes = [i32, i64, i64, i64, op, op, vp, i32, i32, i64, i32, vp,
                                             i64, vp]
        for f in ("mxfp4_qdq_fwd", "mxfp4_ste_bwd", "mxfp4_quant_pack", "mxfp4_grouped_qdq",
                  "mxfp4_quant_pack_kmajor", "mxfp4_dequant", "mxfp8_quant", "mxfp4_version",
                  "mxfp4_grouped_matmul", "mxfp8_quant_kmajor", "mxfp4_mask_to_bool",
                  "mxfp4_qdq_fwd_rows_batch", "mxfp4_ste_bwd_rows_batch"):
            getattr(lib, f).restype = ctypes.c_int32
        lib.mxfp4_last_error.restype = ctypes.c_char_p
        lib.mxfp4_last_error.argtypes = []
        _lib = lib
    return _lib


def library_path() -> str:
    return _LIB_PATH


def mxfp4_last_error() -> str:
    return _load().mxfp4_last_error().decode()


def mxfp4_version() -> int:
    return int(_load().mxfp4_version())


# ------------------------------------------------------------ marshalling

def _rule(rule) -> int:
    if rule in ("floor", FLOOR):
        return FLOOR
    if rule in ("amct", AMCT):
        return AMCT
    raise ValueError(f"rule must be 'floor' or 'amct', got {rule!r}")


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return _BF16
    if t.dtype == torch.float32:
        return _F32
    raise ValueError(f"element dtype must be bfloat16 or float32, got {t.dtype}")


def _shape2d(t: torch.Tensor):
    if t.dim() == 0:
        raise ValueError("x must have at least 1 dimension")
    cols = t.shape[-1]
    rows = t.numel() // cols if cols else 0
    return rows, cols


def _ptr(t, kind=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"expected a torch.Tensor, got {type(t).__name__}")
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU (no CPU path)")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    if kind == "mask" and t.dtype != torch.int32:
        raise ValueError(f"bitmaps are int32 tensors, got {t.dtype}")
    if kind == "u8" and t.dtype != torch.uint8:
        raise ValueError(f"scales / codes are uint8 tensors, got {t.dtype}")
    if kind == "i64" and t.dtype != torch.int64:
        raise ValueError(f"group_list is an int64 tensor, got {t.dtype}")
    if kind == "bool" and t.dtype != torch.bool:
        raise ValueError(f"the expanded mask is a bool tensor, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _desc(x: torch.Tensor, block: int, rule, scale_factor: float) -> _Desc:
    rows, cols = _shape2d(x)
    return _Desc(_dtype(x), int(block), _rule(rule), 0, rows, cols, float(scale_factor), 0)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(status: int, what: str):
    if status == _OK:
        return
    msg = f"{what}: {mxfp4_last_error()}"
    if status in (_EINVAL, _EUNSUPPORTED):
        raise ValueError(msg)
    raise RuntimeError(msg)


def _same_elems(x, *ys):
    for y in ys:
        if y is not None and (y.dtype != x.dtype or y.numel() != x.numel()):
            raise ValueError("outputs must have x's dtype and number of elements")


def _need(t, n: int, what: str):
    """The kernels write (or read) n elements of t: refuse a smaller buffer
    here, since the C ABI takes bare pointers and cannot see its size."""
    if t is not None and t.numel() < n:
        raise ValueError(f"{what} holds {t.numel()} elements; the call needs {n}")


def _block_rows(group_list, rows: int, block: int, group_list_type: int):
    """Block-rows a grouped call produces: exact for a host list (checked by
    _group_list), the bound ceil(rows/block) + groups for a device list."""
    if isinstance(group_list, torch.Tensor) and group_list.is_cuda:
        return grouped_scale_rows_max(rows, block, group_list.numel())
    v = torch.as_tensor(group_list, dtype=torch.int64).reshape(-1).tolist()
    counts = v if group_list_type == 1 else [b - a for a, b in zip([0] + v[:-1], v)]
    return sum(-(-max(int(c), 0) // block) for c in counts)


# ------------------------------------------------------------ entry points

def _group_list(group_list, rows: int, group_list_type: int):
    """group_list on the device as is; a CPU tensor (or sequence) is checked
    first -- counts >= 0 summing to rows (type 1), non-decreasing ends ending
    at rows (type 0), the caller's contract the device cannot check without a
    synchronisation -- then copied to the current device."""
    if group_list is None or (isinstance(group_list, torch.Tensor) and group_list.is_cuda):
        return group_list
    gl = torch.as_tensor(group_list, dtype=torch.int64)
    if gl.dim() != 1 or gl.numel() < 1:
        raise ValueError("group_list must be a non-empty 1-D list of int64")
    v = gl.tolist()
    if group_list_type == 1:
        if min(v) < 0 or sum(v) != rows:
            raise ValueError(f"group counts must be >= 0 and sum to rows={rows}, got sum {sum(v)}")
    elif group_list_type == 0:
        if v[0] < 0 or any(b < a for a, b in zip(v, v[1:])) or v[-1] != rows:
            raise ValueError(f"cumulative group ends must be non-decreasing and end at rows={rows}")
    return gl.to(device=torch.cuda.current_device())



def mxfp4_qdq_fwd(x, axis=ROW, y_row=None, mask_row=None, scales_row=None, y_col=None,
                  mask_col=None, scales_col=None, block=32, rule="floor", scale_factor=6.0):
    """Fused QDQ forward (+ clip bitmap, + E8M0 scales); see include/mxfp4.h."""
    _same_elems(x, y_row, y_col)
    d = _desc(x, block, rule, scale_factor)
    rows, cols, b = d.rows, d.cols, int(block)
    _need(mask_row, rows * -(-cols // 32), "mask_row")
    _need(scales_row, rows * -(-cols // b), "scales_row")
    _need(mask_col, -(-rows // 32) * cols, "mask_col")
    _need(scales_col, -(-rows // b) * cols, "scales_col")
    st = _load().mxfp4_qdq_fwd(ctypes.byref(d), int(axis), _ptr(x), _ptr(y_row),
                               _ptr(mask_row, "mask"), _ptr(scales_row, "u8"), _ptr(y_col),
                               _ptr(mask_col, "mask"), _ptr(scales_col, "u8"), _stream())
    _check(st, "mxfp4_qdq_fwd")


def mxfp4_qdq_fwd_rows_batch(xs, ys=None, masks=None, scales=None, block=32, rule="floor", scale_factor=6.0):
    """Row-wise QDQ forward of up to BATCH_MAX tensors (same dtype) in one
    launch; ys / masks / scales are lists aligned with xs (None entries, or
    None for the whole list, leave that output out)."""
    n = len(xs)
    if not 1 <= n <= BATCH_MAX:
        raise ValueError(f"1 to {BATCH_MAX} tensors per batch, got {n}")
    ys, masks, scales = ([None] * n if v is None else list(v) for v in (ys, masks, scales))
    if not len(ys) == len(masks) == len(scales) == n:
        raise ValueError("ys, masks and scales must have one entry per tensor")
    d = _desc(xs[0], block, rule, scale_factor)
    items = (_RowItem * n)()
    for i, x in enumerate(xs):
        if _dtype(x) != d.dtype:
            raise ValueError("all tensors of a batch must have the same dtype")
        _same_elems(x, ys[i])
        rows, cols = _shape2d(x)
        _need(masks[i], rows * -(-cols // 32), "mask")
        _need(scales[i], rows * -(-cols // int(block)), "scales")
        items[i] = _RowItem(_ptr(x), _ptr(ys[i]), _ptr(masks[i], "mask"), _ptr(scales[i], "u8"), rows, cols)
    _check(_load().mxfp4_qdq_fwd_rows_batch(ctypes.byref(d), n, items, _stream()), "mxfp4_qdq_fwd_rows_batch")


def mxfp4_ste_bwd_rows_batch(grads_out, masks, grads_in, block=32):
    """STE backward of up to BATCH_MAX gradients (same dtype) with ROW
    bitmaps (None: plain STE) in one launch."""
    n = len(grads_out)
    if not 1 <= n <= BATCH_MAX:
        raise ValueError(f"1 to {BATCH_MAX} tensors per batch, got {n}")
    masks = [None] * n if masks is None else list(masks)
    if not len(masks) == len(grads_in) == n:
        raise ValueError("masks and grads_in must have one entry per gradient")
    d = _desc(grads_out[0], block, "floor", 6.0)
    items = (_SteItem * n)()
    for i, g in enumerate(grads_out):
        if _dtype(g) != d.dtype:
            raise ValueError("all tensors of a batch must have the same dtype")
        _same_elems(g, grads_in[i])
        rows, cols = _shape2d(g)
        _need(masks[i], rows * -(-cols // 32), "mask")
        items[i] = _SteItem(_ptr(g), _ptr(masks[i], "mask"), _ptr(grads_in[i]), rows, cols)
    _check(_load().mxfp4_ste_bwd_rows_batch(ctypes.byref(d), n, items, _stream()), "mxfp4_ste_bwd_rows_batch")


def mxfp4_ste_bwd(grad_out, mask, grad_in, layout=ROW, block=32, group_list=None,
                  group_list_type=1):
    """Clipped (mask given) or plain (mask None) STE backward."""
    _same_elems(grad_out, grad_in)
    d = _desc(grad_out, block, "floor", 6.0)
    rows, cols = d.rows, d.cols
    if mask is not None:
        if layout == ROW:
            _need(mask, rows * -(-cols // 32), "mask")
        elif layout == COL:
            _need(mask, -(-rows // 32) * cols, "mask")
        elif layout == GROUPED and group_list is not None:
            nbt = _block_rows(group_list, rows, int(block), group_list_type)
            _need(mask, nbt * (int(block) // 32) * cols, "mask")
    group_list = _group_list(group_list, d.rows, group_list_type)
    n_groups = group_list.numel() if group_list is not None else 0
    st = _load().mxfp4_ste_bwd(ctypes.byref(d), int(layout), _ptr(grad_out), _ptr(mask, "mask"),
                               _ptr(grad_in), _ptr(group_list, "i64"), n_groups,
                               int(group_list_type), _stream())
    _check(st, "mxfp4_ste_bwd")


def mxfp4_mask_to_bool(mask, rows: int, cols: int, layout=ROW, out=None):
    """A ROW or COL saturation bitmap as a bool tensor [rows, cols] (true where
    the forward clipped); ``out`` (bool, contiguous) is filled when given."""
    rows, cols = int(rows), int(cols)
    if layout == ROW:
        _need(mask, rows * -(-cols // 32), "mask")
    elif layout == COL:
        _need(mask, -(-rows // 32) * cols, "mask")
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.bool, device=mask.device)
    _need(out, rows * cols, "out")
    st = _load().mxfp4_mask_to_bool(int(layout), rows, cols, _ptr(mask, "mask"), _ptr(out, "bool"),
                                    _stream())
    _check(st, "mxfp4_mask_to_bool")
    return out


def mxfp4_saturation_mask(x, block=32, rule="floor", scale_factor=6.0, axis=ROW):
    """The pages' saturation mask: a bool tensor of x's shape, true where
    |x| > 6 * 2^k of the element's block (blocks along the last dimension for
    ROW, along the first of the flattened 2-D view for COL).  One forward pass
    writes the bitmap, one more expands it."""
    rows, cols = _shape2d(x)
    if axis == ROW:
        mask = torch.empty(row_mask_shape(rows, cols), dtype=torch.int32, device=x.device)
        mxfp4_qdq_fwd(x, ROW, mask_row=mask, block=block, rule=rule, scale_factor=scale_factor)
    elif axis == COL:
        mask = torch.empty(col_mask_shape(rows, cols), dtype=torch.int32, device=x.device)
        mxfp4_qdq_fwd(x, COL, mask_col=mask, block=block, rule=rule, scale_factor=scale_factor)
    else:
        raise ValueError(f"axis must be ROW or COL, got {axis}")
    out = torch.empty(x.shape, dtype=torch.bool, device=x.device)
    return mxfp4_mask_to_bool(mask, rows, cols, axis, out=out)


def mxfp4_quant_pack(x, codes, scales, y=None, mask=None, block=32, rule="floor",
                     scale_factor=6.0):
    """Packed E2M1 codes (two per byte) + E8M0 scales, row-wise blocks."""
    _same_elems(x, y)
    d = _desc(x, block, rule, scale_factor)
    rows, cols = d.rows, d.cols
    if codes is None or scales is None:
        raise ValueError("codes and scales are required")
    _need(codes, rows * ((cols + 1) // 2), "codes")
    _need(scales, rows * -(-cols // int(block)), "scales")
    _need(mask, rows * -(-cols // 32), "mask")
    st = _load().mxfp4_quant_pack(ctypes.byref(d), _ptr(x), _ptr(codes, "u8"), _ptr(scales, "u8"),
                                  _ptr(y), _ptr(mask, "mask"), _stream())
    _check(st, "mxfp4_quant_pack")


def mxfp4_grouped_qdq(x, group_list, y, mask=None, scales=None, block=32, rule="floor",
                      scale_factor=6.0, group_list_type=1):
    """Grouped column-wise QDQ; group_list = per-group row counts (type 1)
    or cumulative row ends (type 0), int64 on the device."""
    _same_elems(x, y)
    d = _desc(x, block, rule, scale_factor)
    if group_list is None:
        raise ValueError("group_list is required")
    nbt = _block_rows(group_list, d.rows, int(block), group_list_type)
    _need(mask, nbt * (int(block) // 32) * d.cols, "mask")
    _need(scales, nbt * d.cols, "scales")
    group_list = _group_list(group_list, d.rows, group_list_type)
    st = _load().mxfp4_grouped_qdq(ctypes.byref(d), _ptr(x), _ptr(group_list, "i64"),
                                   group_list.numel(), int(group_list_type), _ptr(y),
                                   _ptr(mask, "mask"), _ptr(scales, "u8"), _stream())
    _check(st, "mxfp4_grouped_qdq")


def mxfp4_quant_pack_kmajor(x, codes_t, scales_t, block=32, rule="floor", scale_factor=6.0,
                            group_list=None, group_list_type=1):
    """K-major packed operand of column-wise (group_list None) or grouped
    blocks: codes_t [cols, k_blocks * block / 2] and scales_t [cols, k_blocks]
    uint8, k_blocks being scales_t's second dimension (see kmajor_k_blocks)."""
    rows, cols = _shape2d(x)
    if scales_t is None or scales_t.dim() != 2 or scales_t.shape[0] != cols:
        raise ValueError(f"scales_t must be [cols={cols}, k_blocks]")
    k_blocks = int(scales_t.shape[1])
    if codes_t is None or tuple(codes_t.shape) != (cols, k_blocks * int(block) // 2):
        raise ValueError(f"codes_t must be [{cols}, {k_blocks * int(block) // 2}]")
    d = _desc(x, block, rule, scale_factor)
    group_list = _group_list(group_list, rows, group_list_type)
    n_groups = group_list.numel() if group_list is not None else 0
    st = _load().mxfp4_quant_pack_kmajor(ctypes.byref(d), _ptr(x), _ptr(group_list, "i64"),
                                         n_groups, int(group_list_type), k_blocks,
                                         _ptr(codes_t, "u8"), _ptr(scales_t, "u8"), _stream())
    _check(st, "mxfp4_quant_pack_kmajor")


def mxfp4_dequant(codes, scales, y, block=32):
    """Decode packed codes [rows, ceil(cols/2)] + E8M0 scales [rows,
    ceil(cols/block)] into y [rows, cols] (bfloat16 or float32)."""
    rows, cols = _shape2d(y)
    if codes is None or tuple(codes.shape) != (rows, (cols + 1) // 2):
        raise ValueError(f"codes must be [{rows}, {(cols + 1) // 2}]")
    if scales is None or tuple(scales.shape) != (rows, -(-cols // int(block))):
        raise ValueError(f"scales must be [{rows}, {-(-cols // int(block))}]")
    d = _Desc(_dtype(y), int(block), FLOOR, 0, rows, cols, 6.0, 0)
    st = _load().mxfp4_dequant(ctypes.byref(d), _ptr(codes, "u8"), _ptr(scales, "u8"), _ptr(y),
                               _stream())
    _check(st, "mxfp4_dequant")


_FP8 = {"e4m3": 0, "e5m2": 1}


def mxfp8_quant(x, q, scales, fmt="e4m3", block=32):
    """MXFP8 (OCP MX element rule, blocks of 32 -- or 128 -- along the last
    dim): q uint8 with x's shape, scales uint8 [rows, ceil(cols/block)]."""
    if fmt not in _FP8:
        raise ValueError(f"fmt must be 'e4m3' or 'e5m2', got {fmt!r}")
    rows, cols = _shape2d(x)
    if q is None or q.numel() != x.numel():
        raise ValueError("q must have x's number of elements")
    nb = -(-cols // int(block))
    if scales is None or scales.numel() != rows * nb:
        raise ValueError(f"scales must hold {rows} x {nb} bytes")
    d = _Desc(_dtype(x), int(block), FLOOR, 0, rows, cols, 6.0, 0)
    st = _load().mxfp8_quant(ctypes.byref(d), _FP8[fmt], _ptr(x), _ptr(q, "u8"), _ptr(scales, "u8"),
                             _stream())
    _check(st, "mxfp8_quant")


def mxfp8_quant_kmajor(x, q_t, scales_t, fmt="e4m3", group_list=None, group_list_type=1):
    """K-major MXFP8 of column-wise (group_list None) or grouped 32-row blocks:
    q_t uint8 [cols, k_blocks * 32], scales_t uint8 [cols, k_blocks], k_blocks being
    scales_t's second dimension (see mxfp8_kmajor_k_blocks)."""
    if fmt not in _FP8:
        raise ValueError(f"fmt must be 'e4m3' or 'e5m2', got {fmt!r}")
    rows, cols = _shape2d(x)
    if scales_t is None or scales_t.dim() != 2 or scales_t.shape[0] != cols:
        raise ValueError(f"scales_t must be [cols={cols}, k_blocks]")
    k_blocks = int(scales_t.shape[1])
    if q_t is None or tuple(q_t.shape) != (cols, k_blocks * 32):
        raise ValueError(f"q_t must be [{cols}, {k_blocks * 32}]")
    d = _Desc(_dtype(x), 32, FLOOR, 0, rows, cols, 6.0, 0)
    group_list = _group_list(group_list, rows, group_list_type)
    n_groups = group_list.numel() if group_list is not None else 0
    st = _load().mxfp8_quant_kmajor(ctypes.byref(d), _FP8[fmt], _ptr(x), _ptr(group_list, "i64"), n_groups,
                                    int(group_list_type), k_blocks, _ptr(q_t, "u8"), _ptr(scales_t, "u8"),
                                    _stream())
    _check(st, "mxfp8_quant_kmajor")


MX_FORMATS = {"e4m3": 0, "e5m2": 1, "e2m1": 4}
GROUP_ROWS, GROUP_K = 0, 2


def _operand(data, scales, fmt, block, group_stride=None):
    if fmt not in MX_FORMATS:
        raise ValueError(f"fmt must be one of {sorted(MX_FORMATS)}, got {fmt!r}")
    for t, what in ((data, "data"), (scales, "scales")):
        if t is None or t.dim() not in (2, 3):
            raise ValueError(f"operand {what} must be a 2-D or 3-D uint8 tensor")
    if data.dim() != scales.dim():
        raise ValueError("operand data and scales must have the same rank")
    if group_stride is not None:
        gs, gss = (int(v) for v in group_stride)
    elif data.dim() == 3:
        gs, gss = data.shape[1] * data.shape[2], scales.shape[1] * scales.shape[2]
    else:
        gs, gss = 0, 0
    return _MxOperand(_ptr(data, "u8").value, _ptr(scales, "u8").value, MX_FORMATS[fmt], int(block),
                      data.shape[-1], scales.shape[-1], gs, gss)


def mxfp4_grouped_matmul(a, a_scales, b, b_scales, c, K=None, group_list=None, group_type=GROUP_ROWS,
                         group_list_type=1, a_fmt="e4m3", b_fmt="e2m1", a_block=32, b_block=32,
                         k_blocks=None, b_group_stride=None):
    """Grouped MX matmul C = A . B^T per group (include/mxfp4.h).

    a [M, lda] fp8 codes + a_scales [M, ldas]; b [N, ldb] or [G, N, ldb] codes +
    b_scales of the same rank (b_group_stride = (data bytes, scale bytes) overrides
    the per-group strides); c bf16 / f32 [M, N] (rows-split groups) or [G, M, N]
    (K-split groups).  K defaults to a's row length (rows-split) or the group total
    (K-split, where k_blocks defaults to a's row length / 32)."""
    if c is None or c.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("c must be a bfloat16 or float32 tensor")
    M = a.shape[0]
    ldc = c.shape[-1]
    # rows of every operand array the kernels read (row lengths are checked by
    # the library against ld / ld_scales)
    n_list = 0 if group_list is None else (group_list.numel() if isinstance(group_list, torch.Tensor)
                                           else len(group_list))
    if a_scales is None or a_scales.dim() < 2 or a_scales.shape[-2] < M:
        raise ValueError(f"a_scales must have M={M} rows")
    if b is None or b_scales is None or b.dim() < 2 or b_scales.dim() < 2 or b_scales.shape[-2] != b.shape[-2]:
        raise ValueError("b_scales must have as many rows as b")
    if group_type == GROUP_ROWS and b_group_stride is None and b.dim() == 3:
        if b.shape[0] < max(n_list, 1) or b_scales.shape[0] < max(n_list, 1):
            raise ValueError(f"b and b_scales must hold one matrix per group ({max(n_list, 1)})")
    if group_type == GROUP_ROWS:
        if c.dim() != 2 or c.shape[0] != M:
            raise ValueError(f"c must be [M={M}, N]")
        N = b.shape[-2]
        if K is None:
            K = a.shape[1]
        gl = _group_list(group_list, M, group_list_type)
        kb = 0
    else:
        if group_list is None:
            raise ValueError("groups that split K need a group_list")
        N = b.shape[-2]
        gl_cpu = group_list
        if K is None:
            v = torch.as_tensor(group_list, dtype=torch.int64).tolist() if not (
                isinstance(group_list, torch.Tensor) and group_list.is_cuda) else None
            if v is None:
                raise ValueError("K (the token total) is required with a device group_list")
            K = sum(v) if group_list_type == 1 else v[-1]
        gl = _group_list(gl_cpu, int(K), group_list_type)
        kb = a.shape[1] // 32 if k_blocks is None else int(k_blocks)
        if c.dim() != 3 or c.shape[1] != M:
            raise ValueError(f"c must be [G, M={M}, N]")
    if c.shape[-1] != N:
        raise ValueError(f"c's last dim must be N={N}")
    ng = 0 if gl is None else gl.numel()
    if group_type == GROUP_K and c.shape[0] != ng:
        raise ValueError(f"c must hold one [M, N] matrix per group ({ng})")

    oa = _operand(a, a_scales, a_fmt, a_block)
    ob = _operand(b, b_scales, b_fmt, b_block, b_group_stride)
    out = 1 if c.dtype == torch.float32 else 0
    st = _load().mxfp4_grouped_matmul(int(group_type), M, N, int(K), ctypes.byref(oa), ctypes.byref(ob),
                                      _ptr(gl, "i64"), ng, int(group_list_type), kb, out, _ptr(c), ldc,
                                      _stream())
    _check(st, "mxfp4_grouped_matmul")


# ------------------------------------------------------------ shapes

def row_mask_shape(rows: int, cols: int):
    return rows, -(-cols // 32)


def col_mask_shape(rows: int, cols: int):
    return -(-rows // 32), cols


def grouped_scale_rows_max(rows: int, block: int, num_groups: int) -> int:
    return -(-rows // block) + num_groups


def grouped_mask_rows_max(rows: int, block: int, num_groups: int) -> int:
    return grouped_scale_rows_max(rows, block, num_groups) * (block // 32)


def mxfp8_kmajor_k_blocks(rows: int, num_groups=None, align: bool = True) -> int:
    """k_blocks for mxfp8_quant_kmajor: at least ceil(rows/32) (dense) or
    ceil(rows/32) + num_groups - 1 (grouped).  With align (default) a multiple
    of 16 blocks (512-byte code rows), plus 16 more when the row stride is a
    multiple of 4 KiB.  Measured on MI355X (MoE tokens 32768 x 7168 bf16,
    dense / grouped): k_blocks 1040 takes 142 / 143 us, 1032 152 / 152 us and
    1028 170 us (dense)."""
    nb = -(-rows // 32)
    if num_groups is not None and rows > 0:
        nb += int(num_groups) - 1
    if align:
        nb = -(-nb // 16) * 16
        if nb and (nb * 32) % 4096 == 0:
            nb += 16
    return nb


def kmajor_k_blocks(rows: int, block: int, num_groups=None, align: bool = True) -> int:
    """k_blocks for mxfp4_quant_pack_kmajor: at least ceil(rows/block)
    (dense) or ceil(rows/block) + num_groups - 1 (grouped: the most
    block-rows any split of `rows` into num_groups groups produces).  With
    align (default) it is rounded up so every row of codes_t starts on a
    256-byte boundary (multiples of 16 blocks of 32, 4 blocks of 128; the
    kernel's whole-line stores need at least 128), and a row stride that is a
    multiple of 4 KiB gets 256 more bytes.  The code-row stride decides how
    the workgroups' column lines spread over the memory channels; measured on
    MI355X (bf16, block 32): a 16 KiB stride runs at 4.0 TB/s against 4.9 at
    neighbouring strides, and for the grouped MoE tokens (32768 x 7168, 8
    groups) 256-byte rows take 108.8 us against 117.9 us at the 128-byte
    multiple below them (k_blocks 1040 vs 1032).  The extra block-rows are
    not touched."""
    nb = -(-rows // block)
    if num_groups is not None and rows > 0:
        nb += int(num_groups) - 1
    if align:
        step = 16 if block == 32 else 4
        nb = -(-nb // step) * step
        if nb and (nb * block // 2) % 4096 == 0:
            nb += step
    return nb
