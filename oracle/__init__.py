"""CPU oracle for MXFP4 fake quantization -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package.  The product path (mxfp4_fake_quantization_amd) never does.

Thin ctypes wrapper over liboracle.so (mxfp4_oracle.c).  Arrays are numpy:
bf16 tensors are carried as uint16 bit patterns, fp32 as float32.  Masks are
one bool per element (the pages' saturation mask is a bool tensor).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

F32, BF16, F64 = 0, 1, 2
FLOOR, AMCT = 0, 1

_lib = None


def _load():
    global _lib
    if _lib is None:
        # MXFP4_ORACLE_LIB points the wrapper at another build of the oracle
        # (used by the mutation test, which plants mistakes in a copy).
        path = os.environ.get("MXFP4_ORACLE_LIB") or _build.LIB
        if path == _build.LIB and (not os.path.exists(path)
                                   or os.path.getmtime(path) < os.path.getmtime(_build.SRC)):
            _build.build()
        lib = ctypes.CDLL(path)
        i64, i32, f32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_void_p
        lib.oracle_qdq_rows.argtypes = [i32, i64, i64, i32, i32, f32, vp, vp, vp, vp]
        lib.oracle_qdq_cols.argtypes = [i32, i64, i64, i32, i32, f32, vp, vp, vp, vp]
        lib.oracle_grouped_cols.argtypes = [i32, i64, i64, i32, i32, f32, vp, vp, i32, i32,
                                            vp, vp, vp]
        lib.oracle_ste_bwd.argtypes = [i32, i64, vp, vp, vp]
        lib.oracle_pack_rows.argtypes = [i32, i64, i64, i32, i32, f32, vp, vp, vp]
        lib.oracle_unpack_rows.argtypes = [i32, i64, i64, i32, vp, vp, vp]
        lib.oracle_pack_kmajor.argtypes = [i32, i64, i64, i32, i32, f32, vp, vp, i32, i32, i64,
                                           vp, vp]
        lib.oracle_mxfp8_rows.argtypes = [i32, i64, i64, i32, i32, vp, vp, vp]
        lib.oracle_mxfp8_decode.argtypes = [i32, i64, i64, i32, i32, vp, vp, vp]
        lib.oracle_grouped_matmul.argtypes = [i32, i64, i64, i64, vp, vp, vp, i32, i32, vp]
        lib.oracle_mxfp8_kmajor.argtypes = [i32, i64, i64, i32, vp, vp, i32, i32, i64, vp, vp]
        for fn in ("oracle_qdq_rows", "oracle_qdq_cols", "oracle_grouped_cols",
                   "oracle_ste_bwd", "oracle_pack_rows", "oracle_unpack_rows",
                   "oracle_pack_kmajor", "oracle_mxfp8_rows", "oracle_mxfp8_decode",
                   "oracle_grouped_matmul", "oracle_mxfp8_kmajor"):
            getattr(lib, fn).restype = ctypes.c_int
        _lib = lib
    return _lib


def _dtype_code(x: np.ndarray) -> int:
    if x.dtype == np.float32:
        return F32
    if x.dtype == np.uint16:
        return BF16
    if x.dtype == np.float64:
        return F64
    raise TypeError(f"oracle arrays are float32, uint16 (bf16 bits) or float64, got {x.dtype}")


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _rule_code(rule) -> int:
    if rule in (FLOOR, "floor"):
        return FLOOR
    if rule in (AMCT, "amct"):
        return AMCT
    raise ValueError(f"unknown rule {rule!r}")


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"{what}: oracle returned {rc}")


def qdq_rows(x: np.ndarray, block: int = 32, rule="floor", scale_factor: float = 6.0):
    """Row-wise QDQ of a 2-D array.  Returns (y, clip_bool, e8m0)."""
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    nb = -(-cols // block)
    y = np.empty_like(x)
    clip = np.empty((rows, cols), np.uint8)
    e8 = np.empty((rows, nb), np.uint8)
    _check(_load().oracle_qdq_rows(_dtype_code(x), rows, cols, block, _rule_code(rule),
                                   scale_factor, _ptr(x), _ptr(y), _ptr(clip), _ptr(e8)),
           "qdq_rows")
    return y, clip.astype(bool), e8


def qdq_cols(x: np.ndarray, block: int = 32, rule="floor", scale_factor: float = 6.0):
    """Column-wise QDQ (blocks along dim 0).  Returns (y, clip_bool, e8m0)."""
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    nb = -(-rows // block)
    y = np.empty_like(x)
    clip = np.empty((rows, cols), np.uint8)
    e8 = np.empty((nb, cols), np.uint8)
    _check(_load().oracle_qdq_cols(_dtype_code(x), rows, cols, block, _rule_code(rule),
                                   scale_factor, _ptr(x), _ptr(y), _ptr(clip), _ptr(e8)),
           "qdq_cols")
    return y, clip.astype(bool), e8


def grouped_cols(x: np.ndarray, group_list, block: int = 32, rule="floor",
                 scale_factor: float = 6.0, list_type: int = 1):
    """Grouped column-wise QDQ.  Returns (y, clip_bool, e8m0[block_rows, cols]).

    Rows past the groups' total keep y = x's bits and clip = False (untouched)."""
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    gl = np.ascontiguousarray(np.asarray(group_list, dtype=np.int64))
    counts = gl if list_type == 1 else np.diff(np.concatenate([[0], gl]))
    nbt = int(sum(-(-int(c) // block) for c in counts if c > 0))
    y = x.copy()
    clip = np.zeros((rows, cols), np.uint8)
    e8 = np.empty((nbt, cols), np.uint8)
    _check(_load().oracle_grouped_cols(_dtype_code(x), rows, cols, block, _rule_code(rule),
                                       scale_factor, _ptr(x), _ptr(gl), len(gl), list_type,
                                       _ptr(y), _ptr(clip), _ptr(e8)),
           "grouped_cols")
    return y, clip.astype(bool), e8


def ste_bwd(grad_out: np.ndarray, clip=None):
    """Clipped STE backward (clip given) or plain STE (clip None)."""
    g = np.ascontiguousarray(grad_out)
    out = np.empty_like(g)
    c = None if clip is None else np.ascontiguousarray(clip, dtype=np.uint8)
    _check(_load().oracle_ste_bwd(_dtype_code(g), g.size, _ptr(g), _ptr(c), _ptr(out)),
           "ste_bwd")
    return out


def pack_rows(x: np.ndarray, block: int = 32, rule="floor", scale_factor: float = 6.0):
    """Packed row-wise quantization.  Returns (codes[rows, ceil(cols/2)], e8m0)."""
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    codes = np.empty((rows, (cols + 1) // 2), np.uint8)
    e8 = np.empty((rows, -(-cols // block)), np.uint8)
    _check(_load().oracle_pack_rows(_dtype_code(x), rows, cols, block, _rule_code(rule),
                                    scale_factor, _ptr(x), _ptr(codes), _ptr(e8)),
           "pack_rows")
    return codes, e8


def unpack_rows(codes: np.ndarray, scales: np.ndarray, cols: int, block: int = 32,
                dtype=np.uint16):
    """Decode packed codes + E8M0 scales back to values of `dtype`."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    rows = codes.shape[0]
    y = np.empty((rows, cols), dtype)
    _check(_load().oracle_unpack_rows(_dtype_code(y), rows, cols, block, _ptr(codes),
                                      _ptr(scales), _ptr(y)),
           "unpack_rows")
    return y


def pack_kmajor(x: np.ndarray, block: int = 32, rule="floor", scale_factor: float = 6.0,
                group_list=None, list_type: int = 1, k_blocks=None, fill: int = 0xA5):
    """K-major packed form of column-wise (group_list None) or grouped blocks.

    Returns (codes_t[cols, k_blocks*block/2], scales_t[cols, k_blocks], nbt); block-rows
    at or past nbt keep the `fill` byte (not touched)."""
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    if group_list is None:
        gl, ng = None, 0
        counts = [rows]
    else:
        gl = np.ascontiguousarray(np.asarray(group_list, dtype=np.int64))
        ng = len(gl)
        counts = gl if list_type == 1 else np.diff(np.concatenate([[0], gl]))
    nbt = int(sum(-(-int(c) // block) for c in counts if c > 0))
    kb = nbt if k_blocks is None else int(k_blocks)
    codes = np.full((cols, kb * block // 2), fill, np.uint8)
    scales = np.full((cols, kb), fill, np.uint8)
    _check(_load().oracle_pack_kmajor(_dtype_code(x), rows, cols, block, _rule_code(rule),
                                      scale_factor, _ptr(x), _ptr(gl), ng, list_type, kb,
                                      _ptr(codes), _ptr(scales)),
           "pack_kmajor")
    return codes, scales, nbt


FP8_FORMATS = {"e4m3": 0, "e5m2": 1}


def mxfp8_rows(x: np.ndarray, fmt: str = "e4m3", block: int = 32):
    """Row-wise MXFP8 (blocks of 32 or 128).  Returns (q[rows, cols] bytes,
    e8m0[rows, ceil(cols/block)])."""
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    q = np.empty((rows, cols), np.uint8)
    e8 = np.empty((rows, -(-cols // block)), np.uint8)
    _check(_load().oracle_mxfp8_rows(_dtype_code(x), rows, cols, FP8_FORMATS[fmt], block, _ptr(x), _ptr(q),
                                     _ptr(e8)), "mxfp8_rows")
    return q, e8


def mxfp8_decode(q: np.ndarray, scales: np.ndarray, fmt: str = "e4m3", dtype=np.float32, block: int = 32):
    """Decode MXFP8 bytes + E8M0 scales (one per `block` elements) back to values of `dtype`."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    rows, cols = q.shape
    y = np.empty((rows, cols), dtype)
    _check(_load().oracle_mxfp8_decode(_dtype_code(y), rows, cols, FP8_FORMATS[fmt], block, _ptr(q),
                                       _ptr(scales), _ptr(y)), "mxfp8_decode")
    return y


def mxfp8_kmajor(x: np.ndarray, fmt: str = "e4m3", group_list=None, list_type: int = 1, k_blocks=None,
                 fill: int = 0xA5):
    """K-major MXFP8 of column-wise (group_list None) or grouped 32-row blocks.

    Returns (q_t[cols, k_blocks*32], scales_t[cols, k_blocks], nbt); block-rows at or
    past nbt keep the `fill` byte (not touched)."""
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    if group_list is None:
        gl, ng, counts = None, 0, [rows]
    else:
        gl = np.ascontiguousarray(np.asarray(group_list, dtype=np.int64))
        ng = len(gl)
        counts = gl if list_type == 1 else np.diff(np.concatenate([[0], gl]))
    nbt = int(sum(-(-int(c) // 32) for c in counts if c > 0))
    kb = nbt if k_blocks is None else int(k_blocks)
    q = np.full((cols, kb * 32), fill, np.uint8)
    s = np.full((cols, kb), fill, np.uint8)
    _check(_load().oracle_mxfp8_kmajor(_dtype_code(x), rows, cols, FP8_FORMATS[fmt], _ptr(x), _ptr(gl), ng,
                                       list_type, kb, _ptr(q), _ptr(s)), "mxfp8_kmajor")
    return q, s, nbt


GROUP_M, GROUP_K = 0, 2


def grouped_matmul(left: np.ndarray, right: np.ndarray, group_list=None, group_type: int = GROUP_M,
                   list_type: int = 1, out=None):
    """Grouped matrix product of decoded operand values (float64).

    group_type GROUP_M: left [M, K], right [G, K, N] -> out [M, N] (rows past the groups'
    total keep `out`'s values; a new `out` starts as NaN).
    group_type GROUP_K: left [M, K], right [K, N] -> out [G, M, N].
    group_list None: one group covering the split dimension."""
    left = np.ascontiguousarray(left, dtype=np.float64)
    right = np.ascontiguousarray(right, dtype=np.float64)
    M, K = left.shape
    N = right.shape[-1]
    split = M if group_type == GROUP_M else K
    if group_list is None:
        gl, lt = np.array([split], np.int64), 1
    else:
        gl, lt = np.ascontiguousarray(np.asarray(group_list, dtype=np.int64)), list_type
    G = len(gl)
    if group_type == GROUP_M:
        if right.ndim == 2:
            right = right[None]
        assert right.shape == (G, K, N), (right.shape, G, K, N)
        shape = (M, N)
    else:
        assert right.shape == (K, N), (right.shape, K, N)
        shape = (G, M, N)
    if out is None:
        out = np.full(shape, np.nan)
    assert out.shape == shape and out.dtype == np.float64 and out.flags.c_contiguous
    _check(_load().oracle_grouped_matmul(group_type, M, N, K, _ptr(left), _ptr(right), _ptr(gl), G,
                                         lt, _ptr(out)), "grouped_matmul")
    return out
