"""C-ABI checks that need no GPU: libmxfp4.so loads, exports every function
include/mxfp4.h declares, and rejects bad arguments on the host with the
documented status codes before any HIP call (every call here either fails
validation or has rows*cols == 0, so nothing is launched)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxfp4.h")
LIB = os.path.join(ROOT, "mxfp4_fake_quantization_amd", "libmxfp4.so")

OK, EINVAL, EUNSUP, EHIP = 0, 1, 2, 3
ROW, COL, GROUPED = 1, 2, 4
F32, BF16 = 0, 1
FAKE = 0x10000  # a 16-byte aligned non-NULL address that is never dereferenced


class Desc(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("block", ctypes.c_int32), ("rule", ctypes.c_int32),
                ("reserved0", ctypes.c_int32), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("scale_factor", ctypes.c_float), ("reserved1", ctypes.c_int32)]


class Operand(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("fmt", ctypes.c_int32),
                ("block", ctypes.c_int32), ("ld", ctypes.c_int64), ("ld_scales", ctypes.c_int64),
                ("group_stride", ctypes.c_int64), ("group_stride_scales", ctypes.c_int64)]


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libmxfp4.so is not built (python -m mxfp4_fake_quantization_amd.build)")
    L = ctypes.CDLL(LIB)
    vp, i32 = ctypes.c_void_p, ctypes.c_int32
    dp = ctypes.POINTER(Desc)
    L.mxfp4_qdq_fwd.argtypes = [dp, i32, vp, vp, vp, vp, vp, vp, vp, vp]
    L.mxfp4_ste_bwd.argtypes = [dp, i32, vp, vp, vp, vp, i32, i32, vp]
    L.mxfp4_quant_pack.argtypes = [dp, vp, vp, vp, vp, vp, vp]
    L.mxfp4_grouped_qdq.argtypes = [dp, vp, vp, i32, i32, vp, vp, vp, vp]
    L.mxfp4_quant_pack_kmajor.argtypes = [dp, vp, vp, i32, i32, ctypes.c_int64, vp, vp, vp]
    L.mxfp4_dequant.argtypes = [dp, vp, vp, vp, vp]
    L.mxfp8_quant.argtypes = [dp, i32, vp, vp, vp, vp]
    i64 = ctypes.c_int64
    op = ctypes.POINTER(Operand)
    L.mxfp4_grouped_matmul.argtypes = [i32, i64, i64, i64, op, op, vp, i32, i32, i64, i32, vp, i64, vp]
    L.mxfp8_quant_kmajor.argtypes = [dp, i32, vp, vp, i32, i32, i64, vp, vp, vp]
    L.mxfp4_mask_to_bool.argtypes = [i32, i64, i64, vp, vp, vp]
    L.mxfp4_qdq_fwd_rows_batch.argtypes = [dp, i32, vp, vp]
    L.mxfp4_ste_bwd_rows_batch.argtypes = [dp, i32, vp, vp]
    L.mxfp4_last_error.restype = ctypes.c_char_p
    return L


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\S[^\n(]*?\b(mxfp[48]_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("mxfp4_qdq_fwd", "mxfp4_ste_bwd", "mxfp4_quant_pack", "mxfp4_grouped_qdq",
              "mxfp4_quant_pack_kmajor", "mxfp4_dequant", "mxfp8_quant", "mxfp4_grouped_matmul", "mxfp8_quant_kmajor",
              "mxfp4_mask_to_bool", "mxfp4_qdq_fwd_rows_batch", "mxfp4_ste_bwd_rows_batch",
              "mxfp4_last_error", "mxfp4_version"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert lib.mxfp4_version() == 105


def d(dtype=BF16, block=32, rule=0, rows=64, cols=64, sf=6.0, r0=0, r1=0):
    return Desc(dtype, block, rule, r0, rows, cols, sf, r1)


def P(v=FAKE):
    return ctypes.c_void_p(v)


def fwd(lib, desc, axis=ROW, x=FAKE, yr=FAKE, mr=None, sr=None, yc=None, mc=None, sc=None):
    p = lambda v: None if v is None else P(v)
    return lib.mxfp4_qdq_fwd(ctypes.byref(desc) if desc is not None else None, axis, p(x), p(yr),
                             p(mr), p(sr), p(yc), p(mc), p(sc), None)


def test_qdq_fwd_validation(lib):
    assert fwd(lib, None) == EINVAL
    assert b"desc" in lib.mxfp4_last_error()
    assert fwd(lib, d(block=64)) == EUNSUP
    assert fwd(lib, d(block=16)) == EUNSUP
    assert fwd(lib, d(dtype=7)) == EUNSUP
    assert fwd(lib, d(rule=5)) == EINVAL
    assert fwd(lib, d(rule=1, sf=0.0)) == EINVAL
    assert fwd(lib, d(rule=1, sf=-6.0)) == EINVAL
    assert fwd(lib, d(rows=-1)) == EINVAL
    assert fwd(lib, d(r0=3)) == EINVAL
    assert fwd(lib, d(rows=1 << 40, cols=1 << 40)) == EINVAL       # overflow
    assert fwd(lib, d(), axis=0) == EINVAL
    assert fwd(lib, d(), axis=8) == EINVAL
    assert fwd(lib, d(), x=None) == EINVAL
    assert fwd(lib, d(), x=FAKE + 8) == EINVAL                       # misaligned x
    assert fwd(lib, d(), yr=None) == EINVAL                          # no row output
    assert fwd(lib, d(), yc=FAKE + 64) == EINVAL                     # col output, row axis
    assert fwd(lib, d(), axis=COL, yr=None, yc=None) == EINVAL
    assert fwd(lib, d(), axis=ROW | COL, yr=FAKE + 16, yc=FAKE + 16) == EINVAL   # alias
    assert fwd(lib, d(), axis=ROW | COL, yr=FAKE, yc=FAKE + 32) == EINVAL        # y_row == x (dual)
    assert fwd(lib, d(), axis=ROW, mr=FAKE + 2) == EINVAL            # misaligned bitmap
    assert fwd(lib, d(), axis=ROW, mr=FAKE) == EINVAL                # bitmap aliases x


def test_zero_sized_is_ok_without_launch(lib):
    assert fwd(lib, d(rows=0)) == OK
    assert fwd(lib, d(cols=0), axis=COL, yr=None, yc=FAKE) == OK
    assert fwd(lib, d(rows=0), axis=ROW) == OK                       # in place (y == x)
    assert lib.mxfp4_last_error() == b""


def test_ste_bwd_validation(lib):
    D = d()
    g = lambda *a: lib.mxfp4_ste_bwd(ctypes.byref(D), *a)
    D.rows = 0
    assert g(ROW, P(), P(FAKE + 64), P(FAKE + 128), None, 0, 1, None) == OK
    assert g(3, P(), P(FAKE + 64), P(FAKE + 128), None, 0, 1, None) == EINVAL
    assert g(ROW, None, None, P(FAKE + 128), None, 0, 1, None) == EINVAL
    assert g(ROW, P(), P(FAKE), P(FAKE + 128), None, 0, 1, None) == EINVAL   # mask aliases g
    assert g(GROUPED, P(), P(FAKE + 64), P(FAKE + 128), None, 1, 1, None) == EINVAL
    assert g(GROUPED, P(), P(FAKE + 64), P(FAKE + 128), P(FAKE + 256), 0, 1, None) == EINVAL
    assert g(GROUPED, P(), P(FAKE + 64), P(FAKE + 128), P(FAKE + 256), 2, 7, None) == EINVAL
    assert g(COL, P(), P(FAKE + 4), P(FAKE + 128), None, 0, 1, None) == EINVAL  # col bitmap 16B
    D.block = 64
    assert g(ROW, P(), None, P(FAKE + 128), None, 0, 1, None) == EUNSUP


def test_mask_to_bool_validation(lib):
    m = lib.mxfp4_mask_to_bool
    assert m(ROW, 0, 64, P(), P(FAKE + 1), None) == OK               # empty: nothing launched
    assert m(COL, 64, 0, P(), P(FAKE + 1), None) == OK
    assert m(GROUPED, 4, 4, P(), P(FAKE + 64), None) == EINVAL       # GROUPED needs its group list
    assert m(3, 4, 4, P(), P(FAKE + 64), None) == EINVAL
    assert m(ROW, -1, 4, P(), P(FAKE + 64), None) == EINVAL
    assert m(ROW, 1 << 40, 1 << 30, P(), P(FAKE + 64), None) == EINVAL   # overflow
    assert m(ROW, 4, 4, None, P(FAKE + 64), None) == EINVAL
    assert m(ROW, 4, 4, P(FAKE + 2), P(FAKE + 64), None) == EINVAL   # misaligned bitmap
    assert m(ROW, 4, 4, P(), None, None) == EINVAL
    assert m(ROW, 4, 4, P(), P(FAKE), None) == EINVAL                # out aliases mask
    assert b"alias" in lib.mxfp4_last_error()


class RowItem(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("y", ctypes.c_void_p), ("mask", ctypes.c_void_p),
                ("scales", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64)]


class SteItem(ctypes.Structure):
    _fields_ = [("grad_out", ctypes.c_void_p), ("mask", ctypes.c_void_p), ("grad_in", ctypes.c_void_p),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64)]


def test_batch_validation(lib):
    fb = lambda desc, items: lib.mxfp4_qdq_fwd_rows_batch(
        ctypes.byref(desc) if desc is not None else None, len(items), (RowItem * max(len(items), 1))(*items), None)
    sb = lambda desc, items: lib.mxfp4_ste_bwd_rows_batch(
        ctypes.byref(desc) if desc is not None else None, len(items), (SteItem * max(len(items), 1))(*items), None)
    F = FAKE
    empty = RowItem(F, F + 64, None, None, 0, 64)
    assert fb(d(), [empty]) == OK                                              # empty item: nothing launched
    assert fb(d(), [empty, RowItem(F + 128, F + 192, None, None, 4, 0)]) == OK
    assert fb(d(), []) == EINVAL                                               # n = 0
    assert fb(d(), [empty] * 9) == EINVAL                                      # n > 8
    assert fb(None, [empty]) == EINVAL
    assert fb(d(block=64), [empty]) == EUNSUP
    assert fb(d(), [RowItem(None, None, None, None, 0, 64)]) == OK             # empty: pointers not read
    assert fb(d(), [RowItem(F, None, None, None, 4, 64)]) == EINVAL            # no output
    assert fb(d(), [RowItem(F + 8, F + 64, None, None, 4, 64)]) == EINVAL      # misaligned x
    assert fb(d(), [RowItem(F, F + 64, F + 2, None, 4, 64)]) == EINVAL         # misaligned bitmap
    assert fb(d(), [RowItem(F, F + 64, None, None, -1, 64)]) == EINVAL
    assert fb(d(), [RowItem(F, F + 64, None, None, 4, 64),
                    RowItem(F + 256, F + 64, None, None, 4, 64)]) == EINVAL    # shared y
    assert b"shares" in lib.mxfp4_last_error()
    assert lib.mxfp4_qdq_fwd_rows_batch(ctypes.byref(d()), 1, None, None) == EINVAL
    se = SteItem(F, None, F + 64, 0, 64)
    assert sb(d(), [se]) == OK
    assert sb(d(), [SteItem(F, None, F, 16, 64)]) == OK                        # plain, in place: no launch
    assert sb(d(), [se] * 9) == EINVAL
    assert sb(d(), [SteItem(F, F, F + 64, 4, 64)]) == EINVAL                   # mask aliases grad_out
    assert sb(d(), [SteItem(F, None, F + 64, 4, 64), SteItem(F + 128, None, F + 64, 4, 64)]) == EINVAL
    assert sb(d(), [SteItem(F, None, F + 72, 4, 64)]) == EINVAL                # misaligned grad_in


def test_pack_and_grouped_validation(lib):
    D = d()
    pk = lambda *a: lib.mxfp4_quant_pack(ctypes.byref(D), *a)
    assert pk(P(), None, P(FAKE + 64), None, None, None) == EINVAL           # codes required
    assert pk(P(), P(FAKE + 64), None, None, None, None) == EINVAL           # scales required
    assert pk(P(), P(FAKE + 64), P(FAKE + 64), None, None, None) == EINVAL   # alias
    assert pk(P(), P(FAKE + 72), P(FAKE + 512), None, None, None) == EINVAL  # codes misaligned
    gq = lambda *a: lib.mxfp4_grouped_qdq(ctypes.byref(D), *a)
    assert gq(P(), None, 8, 1, P(FAKE + 64), None, None, None) == EINVAL
    assert gq(P(), P(FAKE + 4), 8, 1, P(FAKE + 64), None, None, None) == EINVAL
    assert gq(P(), P(FAKE + 1024), 0, 1, P(FAKE + 64), None, None, None) == EINVAL
    assert gq(P(), P(FAKE + 1024), 8, 2, P(FAKE + 64), None, None, None) == EINVAL
    assert gq(P(), P(FAKE + 1024), 8, 1, None, None, None, None) == EINVAL
    assert gq(P(), P(FAKE + 1024), 8, 1, P(FAKE + 1024), None, None, None) == EINVAL  # y aliases list
    D.rows = 0
    assert gq(P(), P(FAKE + 1024), 8, 1, P(FAKE), None, None, None) == OK


def test_kmajor_and_dequant_validation(lib):
    D = d(rows=70, cols=64)
    km = lambda *a: lib.mxfp4_quant_pack_kmajor(ctypes.byref(D), *a)
    x, c, s, gl = P(), P(FAKE + 4096), P(FAKE + 8192), P(FAKE + 12288)
    assert km(x, None, 0, 1, 2, c, s, None) == EINVAL                  # 70 rows need 3 blocks
    assert b"k_blocks" in lib.mxfp4_last_error()
    assert km(x, gl, 4, 1, 5, c, s, None) == EINVAL                    # grouped: 3 + 4 - 1
    assert km(x, gl, 0, 1, 9, c, s, None) == EINVAL                    # num_groups < 1
    assert km(x, gl, 4, 3, 9, c, s, None) == EINVAL                    # list type
    assert km(x, P(FAKE + 12292), 4, 1, 9, c, s, None) == EINVAL       # list misaligned
    assert km(x, None, 0, 1, 3, P(FAKE + 4100), s, None) == EINVAL     # codes misaligned
    assert km(x, None, 0, 1, 3, None, s, None) == EINVAL
    assert km(x, None, 0, 1, 3, c, None, None) == EINVAL
    assert km(x, None, 0, 1, 3, c, c, None) == EINVAL                  # alias
    assert km(x, None, 0, 1, 1 << 60, c, s, None) == EINVAL            # size overflow
    D.block = 64
    assert km(x, None, 0, 1, 3, c, s, None) == EUNSUP
    D.block, D.rows = 32, 0
    assert km(x, gl, 4, 1, 0, c, s, None) == OK                        # nothing to do
    dq = lambda *a: lib.mxfp4_dequant(ctypes.byref(D), *a)
    D.rows = 4
    assert dq(None, s, x, None) == EINVAL
    assert dq(c, None, x, None) == EINVAL
    assert dq(c, s, None, None) == EINVAL
    assert dq(c, s, P(FAKE + 8), None) == EINVAL                       # y misaligned
    assert dq(c, c, x, None) == EINVAL                                 # alias
    D.dtype = 5
    assert dq(c, s, x, None) == EUNSUP
    D.dtype, D.rows = BF16, 0
    assert dq(c, s, x, None) == OK


def test_mxfp8_validation(lib):
    D = d(rows=8, cols=64)
    m8 = lambda *a: lib.mxfp8_quant(ctypes.byref(D), *a)
    x, q, s = P(), P(FAKE + 4096), P(FAKE + 8192)
    assert m8(2, x, q, s, None) == EINVAL                   # unknown fmt
    assert m8(0, None, q, s, None) == EINVAL
    assert m8(0, x, None, s, None) == EINVAL
    assert m8(0, x, q, None, None) == EINVAL
    assert m8(0, x, P(FAKE + 4100), s, None) == EINVAL     # q misaligned
    assert m8(0, x, q, q, None) == EINVAL                   # alias
    D.block = 64
    assert m8(0, x, q, s, None) == EUNSUP                   # blocks of 32 or 128
    D.block, D.rows = 128, 0
    assert m8(1, x, q, s, None) == OK                       # block 128 accepted (nothing to do)
    D.block = 32
    assert m8(1, x, q, s, None) == OK


def test_grouped_matmul_validation(lib):
    """Every bad argument is refused on the host; M == 0 or N == 0 returns OK
    without a launch."""
    def ops(afmt=0, bfmt=4, ab=32, bb=32, lda=256, ldas=8, ldb=128, ldbs=8, gs=0, gss=0, adata=FAKE):
        return (Operand(adata, FAKE + 65536, afmt, ab, lda, ldas, 0, 0),
                Operand(FAKE + 131072, FAKE + 196608, bfmt, bb, ldb, ldbs, gs, gss))

    def mm(gt=0, M=64, N=64, K=256, a=None, b=None, gl=None, ng=0, lt=1, kb=0, out=0, c=FAKE + 262144,
           ldc=64):
        if a is None:
            a, b = ops()
        return lib.mxfp4_grouped_matmul(gt, M, N, K, ctypes.byref(a), ctypes.byref(b),
                                        None if gl is None else P(gl), ng, lt, kb, out, P(c), ldc, None)

    assert mm(gt=1) == EINVAL                                   # unknown group_type
    assert mm(K=100) == EINVAL                                  # K not a multiple of 32
    assert mm(K=0) == EUNSUP                                    # rows split over an empty K
    assert mm(M=-1) == EINVAL
    assert mm(*(), **{"a": ops(afmt=4)[0], "b": ops()[1]}) == EUNSUP   # A must be fp8
    assert mm(a=ops()[0], b=ops(bfmt=2)[1]) == EUNSUP           # unknown B format
    assert mm(a=ops(ab=64)[0], b=ops()[1]) == EUNSUP            # scale block 64
    assert mm(a=ops(lda=255)[0], b=ops()[1]) == EINVAL          # ld not a multiple of 16
    assert mm(a=ops(lda=240)[0], b=ops()[1]) == EINVAL          # ld shorter than K bytes
    assert mm(a=ops()[0], b=ops(ldb=112)[1]) == EINVAL          # fp4 row is K/2 bytes
    assert mm(a=ops(ldas=7)[0], b=ops()[1]) == EINVAL           # too few scale bytes
    assert mm(a=ops(adata=FAKE + 8)[0], b=ops()[1]) == EINVAL   # misaligned data
    assert mm(a=ops()[0], b=ops(gs=8)[1]) == EINVAL             # group stride not 16-aligned
    assert mm(out=2) == EUNSUP
    assert mm(c=FAKE + 1) == EINVAL                             # misaligned output
    assert mm(ldc=63) == EINVAL
    assert mm(gl=FAKE, ng=0) == EINVAL                          # list without groups
    assert mm(gl=FAKE, ng=2, lt=3) == EINVAL
    assert mm(gt=2, gl=None, kb=8) == EINVAL                    # K-split needs a list
    a, b = ops(ab=128, bb=128)
    assert mm(gt=2, a=a, b=b, gl=FAKE, ng=1, kb=8) == EUNSUP     # K-split needs blocks of 32
    assert mm(gt=2, gl=FAKE, ng=1, kb=8, a=ops(lda=240)[0], b=ops()[1]) == EINVAL  # ld < k_blocks*32
    assert mm(M=0) == OK and mm(N=0) == OK                       # nothing to launch


def test_mxfp8_kmajor_validation(lib):
    D = d(rows=100, cols=64)
    km = lambda fmt, x, gl, ng, lt, kb, q, s: lib.mxfp8_quant_kmajor(ctypes.byref(D), fmt, x, gl, ng, lt, kb, q, s, None)
    x, q, s = P(), P(FAKE + 65536), P(FAKE + 131072)
    assert km(2, x, None, 0, 1, 4, q, s) == EINVAL                      # unknown fmt
    assert km(0, x, None, 0, 1, 3, q, s) == EINVAL                      # needs 4 block-rows
    assert km(0, x, P(FAKE), 3, 1, 5, q, s) == EINVAL                   # grouped: needs 4 + 3 - 1
    assert km(0, x, P(FAKE), 0, 1, 9, q, s) == EINVAL                   # list without groups
    assert km(0, x, P(FAKE), 2, 2, 9, q, s) == EINVAL                   # list type
    assert km(0, x, None, 0, 1, 4, P(FAKE + 65537), s) == EINVAL        # q misaligned
    assert km(0, x, None, 0, 1, 4, q, q) == EINVAL                      # alias
    D.block = 128
    assert km(0, x, None, 0, 1, 4, q, s) == EUNSUP
    D.block, D.rows = 32, 0
    assert km(0, x, None, 0, 1, 0, q, s) == OK                          # nothing to do


def test_python_binding_refuses_cpu_tensors():
    import torch
    import mxfp4_fake_quantization_amd as M
    x = torch.zeros(4, 32, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        M.mxfp4_qdq_fwd(x, M.ROW, y_row=torch.empty_like(x))


def test_cpu_group_list_is_validated_before_any_gpu_work():
    """A CPU group_list is checked on the host (the device cannot check the
    sum without a synchronisation): counts must be >= 0 and sum to rows."""
    import mxfp4_fake_quantization_amd as M
    with pytest.raises(ValueError, match="sum to rows"):
        M._group_list([10, 20], 31, 1)
    with pytest.raises(ValueError, match="sum to rows"):
        M._group_list([40, -9], 31, 1)
    with pytest.raises(ValueError, match="non-decreasing"):
        M._group_list([20, 10, 31], 31, 0)
    with pytest.raises(ValueError, match="non-decreasing"):
        M._group_list([10, 30], 31, 0)
    with pytest.raises(ValueError):
        M._group_list([], 0, 1)


ROWS_SET = [0, 1, 31, 32, 33, 127, 128, 300, 4095, 4096, 16384, 28672, 32768, 32769, 65536, 131072]


@pytest.mark.parametrize("block", [32, 128])
@pytest.mark.parametrize("groups", [None, 1, 3, 8, 40])
def test_kmajor_k_blocks_rule(block, groups):
    """kmajor_k_blocks: the smallest k_blocks >= the most block-rows the
    blocking can produce whose codes_t row is a whole number of 256-byte units
    and not a multiple of 4 KiB (align=False: that minimum itself)."""
    import mxfp4_fake_quantization_amd as M
    bpb = block // 2                      # code bytes per block
    for rows in ROWS_SET:
        need = -(-rows // block) + ((groups - 1) if groups and rows else 0)
        assert M.kmajor_k_blocks(rows, block, groups, align=False) == need
        kb = M.kmajor_k_blocks(rows, block, groups)
        if need == 0:
            assert kb == 0
            continue
        ok = lambda k: (k * bpb) % 256 == 0 and (k * bpb) % 4096 != 0
        assert kb >= need and ok(kb)
        assert not any(ok(k) for k in range(need, kb))
        assert kb % (8 if block == 32 else 2) == 0          # whole 128-byte code lines
        assert kb % 8 == 0 or block == 128                  # 8-byte aligned scale rows


@pytest.mark.parametrize("groups", [None, 1, 3, 8, 40])
def test_mxfp8_kmajor_k_blocks_rule(groups):
    """mxfp8_kmajor_k_blocks: the same with 512-byte code rows (32 bytes per
    block of 32)."""
    import mxfp4_fake_quantization_amd as M
    for rows in ROWS_SET:
        need = -(-rows // 32) + ((groups - 1) if groups and rows else 0)
        assert M.mxfp8_kmajor_k_blocks(rows, groups, align=False) == need
        kb = M.mxfp8_kmajor_k_blocks(rows, groups)
        if need == 0:
            assert kb == 0
            continue
        ok = lambda k: (k * 32) % 512 == 0 and (k * 32) % 4096 != 0
        assert kb >= need and ok(kb)
        assert not any(ok(k) for k in range(need, kb))


def test_k_blocks_of_the_measured_shapes():
    """The values the measured stride tables rest on (MoE tokens 32768 rows in
    8 groups, the 28672-row weight)."""
    import mxfp4_fake_quantization_amd as M
    assert M.kmajor_k_blocks(32768, 32) == M.kmajor_k_blocks(32768, 32, 8) == 1040
    assert M.kmajor_k_blocks(28672, 32) == 896
    assert M.kmajor_k_blocks(28672, 128) == 224
    assert M.mxfp8_kmajor_k_blocks(32768) == M.mxfp8_kmajor_k_blocks(32768, 8) == 1040
