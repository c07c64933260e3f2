"""GPU parity at the largest sizes: tensors of more than 2^31 elements (byte
offsets past 4 GiB), so every 64-bit index and address path of each entry
point is exercised.  Inputs are drawn on the device with a seeded torch
generator (bf16 N(0, 1) rows scaled by per-row powers of two, sparse
outliers, all-zero blocks); the oracle recomputes sampled rows or columns
from host copies of exactly those inputs, including the rows and columns
that straddle element 2^31, and the results must agree bit for bit (the
matmul: within the matrix-core bound of mx_tolerance)."""
import numpy as np
import pytest
import torch

from gpu_util import host, unpack_col_bitmap, unpack_grouped_bitmap, unpack_row_bitmap
from mx_tolerance import mx_matmul_bound

pytestmark = pytest.mark.gpu

M = None
BIG = 1 << 31


@pytest.fixture(scope="module", autouse=True)
def lib():
    global M
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mxfp4_fake_quantization_amd as mod
    mod._load()
    M = mod
    yield
    torch.cuda.empty_cache()


def big_bf16(rows, cols, seed, chunk_elems=1 << 28):
    """bf16 [rows, cols] on the device: N(0, 1) times 2^e per row (e uniform in
    [-40, 20]), every 1009th element x 300, every 97th 32-element block zero."""
    assert rows * cols > BIG
    gen = torch.Generator(device="cuda").manual_seed(seed)
    x = torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda")
    step = max(1, chunk_elems // cols)
    for r0 in range(0, rows, step):
        n = min(step, rows - r0)
        e = torch.randint(-40, 21, (n, 1), generator=gen, device="cuda").float()
        x[r0:r0 + n] = (torch.randn((n, cols), generator=gen, device="cuda") * torch.exp2(e)).to(torch.bfloat16)
    flat = x.view(-1)
    flat[::1009] *= 300
    if cols % 32 == 0:
        flat.view(-1, 32)[::97] = 0
    return x


def sample_rows(rows, cols, seed, k=6):
    """Row indices: first, last, those holding elements 2^31 - 1 and 2^31, and k random."""
    r = {0, rows - 1, (BIG - 1) // cols, BIG // cols, min(rows - 1, BIG // cols + 1)}
    r.update(np.random.default_rng(seed).choice(rows, k, replace=False).tolist())
    return np.array(sorted(r), dtype=np.int64)


def sample_cols(cols, seed, k=6):
    c = {0, cols - 1}
    c.update(np.random.default_rng(seed).choice(cols, k, replace=False).tolist())
    return np.array(sorted(c), dtype=np.int64)


def rows_of(t, ri):
    return host(t[torch.from_numpy(ri).cuda()])


def cols_of(t, ci):
    return np.ascontiguousarray(host(t[:, torch.from_numpy(ci).cuda()]))


@pytest.mark.parametrize("cols", [32768, 32760], ids=["flat", "ragged_rows"])
def test_row_fwd_and_ste_beyond_int32(oracle, cols):
    """Row-wise forward (y + bitmap) and clipped STE over > 2^31 elements, in
    the flat layout (cols % 32 == 0) and the row walk (cols % 32 != 0)."""
    rows = BIG // cols + 17
    x = big_bf16(rows, cols, 1)
    y = torch.empty_like(x)
    nw = -(-cols // 32)
    m = torch.empty((rows, nw), dtype=torch.int32, device="cuda")
    M.mxfp4_qdq_fwd(x, M.ROW, y_row=y, mask_row=m)
    g = torch.randn((rows, cols), generator=torch.Generator(device="cuda").manual_seed(2), device="cuda",
                    dtype=torch.float32).to(torch.bfloat16)
    gi = torch.empty_like(g)
    M.mxfp4_ste_bwd(g, m, gi, layout=M.ROW)
    torch.cuda.synchronize()
    ri = sample_rows(rows, cols, 3)
    xs = rows_of(x, ri)
    yo, clip, _ = oracle.qdq_rows(xs, 32)
    assert np.array_equal(rows_of(y, ri), yo)
    bits, clean = unpack_row_bitmap(rows_of(m, ri), cols)
    assert np.array_equal(bits, clip) and clean
    assert np.array_equal(rows_of(gi, ri), oracle.ste_bwd(rows_of(g, ri), clip))
    assert clip.any()


@pytest.mark.parametrize("block", [32, 128])
def test_pack_beyond_int32(oracle, block):
    """Row-wise packed codes + E8M0 scales + y in one pass over > 2^31 elements."""
    cols = 16384
    rows = BIG // cols + 33
    x = big_bf16(rows, cols, 4)
    codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device="cuda")
    sc = torch.empty((rows, cols // block), dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    M.mxfp4_quant_pack(x, codes, sc, y=y, block=block)
    torch.cuda.synchronize()
    ri = sample_rows(rows, cols, 5)
    xs = rows_of(x, ri)
    co, so = oracle.pack_rows(xs, block)
    assert np.array_equal(rows_of(codes, ri), co)
    assert np.array_equal(rows_of(sc, ri), so)
    assert np.array_equal(rows_of(y, ri), oracle.qdq_rows(xs, block)[0])


def test_dual_beyond_int32(oracle):
    """Row and column views in one launch over > 2^31 elements, with a short
    last block-row; sampled rows (row view) and columns (column view)."""
    cols = 8192
    rows = BIG // cols + 6          # 262150: the last column block is 6 rows
    x = big_bf16(rows, cols, 6)
    yr = torch.empty_like(x)
    yc = torch.empty_like(x)
    mr = torch.empty((rows, cols // 32), dtype=torch.int32, device="cuda")
    mc = torch.empty((-(-rows // 32), cols), dtype=torch.int32, device="cuda")
    M.mxfp4_qdq_fwd(x, M.ROW | M.COL, y_row=yr, mask_row=mr, y_col=yc, mask_col=mc)
    torch.cuda.synchronize()
    ri = sample_rows(rows, cols, 7)
    yo, clip, _ = oracle.qdq_rows(rows_of(x, ri), 32)
    assert np.array_equal(rows_of(yr, ri), yo)
    assert np.array_equal(unpack_row_bitmap(rows_of(mr, ri), cols)[0], clip)
    ci = sample_cols(cols, 8)
    yo, clip, _ = oracle.qdq_cols(cols_of(x, ci), 32)
    assert np.array_equal(cols_of(yc, ci), yo)
    bits, clean = unpack_col_bitmap(cols_of(mc, ci), rows)
    assert np.array_equal(bits, clip) and clean


def test_grouped_and_ste_beyond_int32(oracle):
    """Grouped column-wise QDQ (y, GROUPED bitmap, scales) and the grouped
    STE over > 2^31 elements in 8 groups of multinomial size; sampled columns."""
    cols = 7168
    rows = BIG // cols + 100
    counts = np.random.default_rng(9).multinomial(rows, [1 / 8] * 8).astype(np.int64)
    x = big_bf16(rows, cols, 10)
    y = torch.empty_like(x)
    mask = torch.empty((M.grouped_mask_rows_max(rows, 32, 8), cols), dtype=torch.int32, device="cuda")
    sc = torch.empty((M.grouped_scale_rows_max(rows, 32, 8), cols), dtype=torch.uint8, device="cuda")
    gl = torch.from_numpy(counts).cuda()
    M.mxfp4_grouped_qdq(x, gl, y, mask=mask, scales=sc)
    g = torch.randn((rows, cols), generator=torch.Generator(device="cuda").manual_seed(11), device="cuda",
                    dtype=torch.float32).to(torch.bfloat16)
    gi = torch.empty_like(g)
    M.mxfp4_ste_bwd(g, mask, gi, layout=M.GROUPED, group_list=gl)
    torch.cuda.synchronize()
    ci = sample_cols(cols, 12)
    yo, clip, eo = oracle.grouped_cols(cols_of(x, ci), counts, 32)
    assert np.array_equal(cols_of(y, ci), yo)
    nbt = eo.shape[0]
    assert np.array_equal(cols_of(sc, ci)[:nbt], eo)
    bits, clean = unpack_grouped_bitmap(cols_of(mask, ci)[:nbt], rows, counts, 32)
    assert np.array_equal(bits, clip) and clean
    assert np.array_equal(cols_of(gi, ci), oracle.ste_bwd(cols_of(g, ci), clip))


@pytest.mark.parametrize("grouped", [False, True], ids=["dense", "grouped"])
def test_kmajor_beyond_int32(oracle, grouped):
    """K-major packed operand of column-wise or grouped blocks of a > 2^31
    element tensor; sampled columns (whole K runs of codes and scales)."""
    cols = 7168
    rows = BIG // cols + 100
    x = big_bf16(rows, cols, 13)
    counts = np.random.default_rng(14).multinomial(rows, [1 / 8] * 8).astype(np.int64) if grouped else None
    kb = M.kmajor_k_blocks(rows, 32, 8 if grouped else None)
    codes = torch.empty((cols, kb * 16), dtype=torch.uint8, device="cuda")
    sc = torch.empty((cols, kb), dtype=torch.uint8, device="cuda")
    M.mxfp4_quant_pack_kmajor(x, codes, sc, block=32,
                              group_list=None if counts is None else torch.from_numpy(counts).cuda())
    torch.cuda.synchronize()
    ci = sample_cols(cols, 15)
    co, so, nbt = oracle.pack_kmajor(cols_of(x, ci), 32, group_list=counts, k_blocks=kb)
    cit = torch.from_numpy(ci).cuda()
    assert np.array_equal(host(codes[cit])[:, : nbt * 16], co[:, : nbt * 16])
    assert np.array_equal(host(sc[cit])[:, :nbt], so[:, :nbt])


def test_dequant_beyond_int32(oracle):
    """Decode of random packed codes and E8M0 bytes into > 2^31 bf16 values."""
    cols = 32768
    rows = BIG // cols + 9
    gen = torch.Generator(device="cuda").manual_seed(16)
    codes = torch.randint(0, 256, (rows, cols // 2), generator=gen, device="cuda", dtype=torch.uint8)
    sc = torch.randint(60, 200, (rows, cols // 32), generator=gen, device="cuda", dtype=torch.uint8)
    y = torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda")
    M.mxfp4_dequant(codes, sc, y, block=32)
    torch.cuda.synchronize()
    ri = sample_rows(rows, cols, 17)
    yo = oracle.unpack_rows(rows_of(codes, ri), rows_of(sc, ri), cols, 32)
    assert np.array_equal(rows_of(y, ri), yo)


def test_mxfp8_rows_and_kmajor_beyond_int32(oracle):
    """MXFP8 row-wise (grad_output) and grouped K-major (TN operand) over a
    > 2^31 element tensor; sampled rows and columns."""
    cols = 7168
    rows = BIG // cols + 100
    x = big_bf16(rows, cols, 18)
    q = torch.empty((rows, cols), dtype=torch.uint8, device="cuda")
    s = torch.empty((rows, cols // 32), dtype=torch.uint8, device="cuda")
    M.mxfp8_quant(x, q, s)
    counts = np.random.default_rng(19).multinomial(rows, [1 / 8] * 8).astype(np.int64)
    kb = M.mxfp8_kmajor_k_blocks(rows, 8)
    qt = torch.empty((cols, kb * 32), dtype=torch.uint8, device="cuda")
    st = torch.empty((cols, kb), dtype=torch.uint8, device="cuda")
    M.mxfp8_quant_kmajor(x, qt, st, group_list=torch.from_numpy(counts).cuda())
    torch.cuda.synchronize()
    ri = sample_rows(rows, cols, 20)
    qo, so = oracle.mxfp8_rows(rows_of(x, ri))
    assert np.array_equal(rows_of(q, ri), qo)
    assert np.array_equal(rows_of(s, ri), so)
    ci = sample_cols(cols, 21)
    qo, so, nbt = oracle.mxfp8_kmajor(cols_of(x, ci), group_list=counts, k_blocks=kb)
    cit = torch.from_numpy(ci).cuda()
    assert np.array_equal(host(qt[cit])[:, : nbt * 32], qo[:, : nbt * 32])
    assert np.array_equal(host(st[cit])[:, :nbt], so[:, :nbt])


def test_matmul_operand_beyond_4gib(oracle):
    """Grouped MX matmul whose MXFP8 A operand spans more than 4 GiB (64-bit
    tile bases) in two row groups: random finite E4M3 codes x random E2M1
    codes, sampled output rows (those past 4 GiB included) within the
    matrix-core bound."""
    K, N = 7168, 256
    Mr = (1 << 32) // K + 300
    gen = torch.Generator(device="cuda").manual_seed(22)
    a = torch.randint(0, 256, (Mr, K), generator=gen, device="cuda", dtype=torch.uint8)
    a[a == 0x7F] = 0x7E                               # no E4M3 NaN codes
    a[a == 0xFF] = 0xFE
    sa = torch.randint(118, 130, (Mr, K // 32), generator=gen, device="cuda", dtype=torch.uint8)
    b = torch.randint(0, 256, (2, N, K // 2), generator=gen, device="cuda", dtype=torch.uint8)
    sb = torch.randint(118, 130, (2, N, K // 32), generator=gen, device="cuda", dtype=torch.uint8)
    counts = [Mr // 3, Mr - Mr // 3]
    c = torch.empty((Mr, N), dtype=torch.float32, device="cuda")
    M.mxfp4_grouped_matmul(a, sa, b, sb, c, group_list=counts)
    torch.cuda.synchronize()
    ri = np.array(sorted({0, counts[0] - 1, counts[0], (1 << 31) // K, (1 << 32) // K,
                          (1 << 32) // K + 1, Mr - 1}
                         | set(np.random.default_rng(23).choice(Mr, 8, replace=False).tolist())))
    A = oracle.mxfp8_decode(rows_of(a, ri), rows_of(sa, ri), "e4m3", np.float64)
    got = rows_of(c, ri).astype(np.float64)
    for gidx in range(2):
        sel = (ri >= counts[0]) if gidx else (ri < counts[0])
        Bv = oracle.unpack_rows(host(b[gidx]), host(sb[gidx]), K, 32, np.float64)   # [N, K]
        exp = oracle.grouped_matmul(A[sel], Bv.T.copy()[None], None, oracle.GROUP_M)
        bound = mx_matmul_bound(A[sel], Bv) + 1e-30
        ratio = np.abs(got[sel] - exp) / bound
        assert (ratio <= 1).all(), f"group {gidx}: worst error / bound {ratio.max():.3g}"
