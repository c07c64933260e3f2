"""Full-size GPU parity for the five workloads: every output element of the
launch the benchmark times, compared with the oracle bit for bit (0 ULP).

- tiny QAT (fp32 32x64 weight, 4x64 input): forward y + bitmap, clipped STE
  of a ones gradient;
- weight_4k (bf16 4096x4096, outliers, zero blocks, planted blocks): forward
  y + bitmap + scales, clipped STE of the upstream gradient;
- act_dual (bf16 16384x8192 Student-t): one dual-direction launch, y_row,
  y_col, both bitmaps and both scale arrays;
- moe_grouped (bf16 32768x7168, 8 expert groups): grouped column-wise y,
  GROUPED bitmap and scales; the GROUPED-layout STE; the grouped K-major
  operand;
- weight_pack (bf16 28672x8192): packed codes + E8M0 bytes at blocks 32 and
  128, decoded on the GPU and compared with the QDQ values; the K-major
  operand.
Padding bits of every bitmap must be zero and block-rows past the grouped
blocking untouched."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import dev, host, unpack_col_bitmap, unpack_grouped_bitmap, unpack_row_bitmap

pytestmark = pytest.mark.gpu

M = None
FILL = 0x5A


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


def _eq(got, want, what):
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        raise AssertionError(f"{what}: {len(bad)} mismatches, first at {bad[:3].tolist()}")


def test_tiny_qat_full(oracle):
    w, xin = W.tiny_qat(0)
    for a in (w, xin):
        rows, cols = a.shape
        y = torch.empty(a.shape, dtype=torch.float32, device="cuda")
        m = torch.empty((rows, cols // 32), dtype=torch.int32, device="cuda")
        s = torch.empty((rows, cols // 32), dtype=torch.uint8, device="cuda")
        M.mxfp4_qdq_fwd(dev(a), M.ROW, y_row=y, mask_row=m, scales_row=s)
        gi = torch.empty_like(y)
        M.mxfp4_ste_bwd(torch.ones_like(y), m, gi, layout=M.ROW)
        torch.cuda.synchronize()
        yo, clip, eo = oracle.qdq_rows(a, 32)
        _eq(host(y).view(np.uint32), yo.view(np.uint32), "y")
        bits, clean = unpack_row_bitmap(host(m), cols)
        _eq(bits, clip, "bitmap")
        assert clean
        _eq(host(s), eo, "scales")
        _eq(host(gi).view(np.uint32), oracle.ste_bwd(np.ones_like(a), clip).view(np.uint32), "g_in")


def test_weight_4k_full(oracle):
    x, g, manifest = W.weight_4k()
    rows, cols = x.shape
    y = torch.empty(x.shape, dtype=torch.bfloat16, device="cuda")
    m = torch.empty((rows, cols // 32), dtype=torch.int32, device="cuda")
    s = torch.empty((rows, cols // 32), dtype=torch.uint8, device="cuda")
    M.mxfp4_qdq_fwd(dev(x), M.ROW, y_row=y, mask_row=m, scales_row=s)
    gi = torch.empty_like(y)
    M.mxfp4_ste_bwd(dev(g), m, gi, layout=M.ROW)
    torch.cuda.synchronize()
    yo, clip, eo = oracle.qdq_rows(x, 32)
    _eq(host(y), yo, "y")
    bits, clean = unpack_row_bitmap(host(m), cols)
    _eq(bits, clip, "bitmap")
    assert clean and clip.any() and len(manifest) > 0
    _eq(host(s), eo, "scales")
    _eq(host(gi), oracle.ste_bwd(g, clip), "g_in")


def test_act_dual_full(oracle):
    x = W.act_dual()
    rows, cols = x.shape
    yr = torch.empty(x.shape, dtype=torch.bfloat16, device="cuda")
    yc = torch.empty_like(yr)
    mr = torch.empty((rows, cols // 32), dtype=torch.int32, device="cuda")
    mc = torch.empty((rows // 32, cols), dtype=torch.int32, device="cuda")
    sr = torch.empty((rows, cols // 32), dtype=torch.uint8, device="cuda")
    sc = torch.empty((rows // 32, cols), dtype=torch.uint8, device="cuda")
    M.mxfp4_qdq_fwd(dev(x), M.ROW | M.COL, y_row=yr, mask_row=mr, scales_row=sr,
                    y_col=yc, mask_col=mc, scales_col=sc)
    torch.cuda.synchronize()
    yo, co, eo = oracle.qdq_rows(x, 32)
    _eq(host(yr), yo, "y_row")
    bits, clean = unpack_row_bitmap(host(mr), cols)
    _eq(bits, co, "mask_row")
    assert clean
    _eq(host(sr), eo, "scales_row")
    del yo, co, eo, bits
    yo, co, eo = oracle.qdq_cols(x, 32)
    _eq(host(yc), yo, "y_col")
    bits, clean = unpack_col_bitmap(host(mc), rows)
    _eq(bits, co, "mask_col")
    assert clean
    _eq(host(sc), eo, "scales_col")


def test_moe_grouped_full(oracle):
    x, counts = W.moe_grouped()
    rows, cols = x.shape
    G = len(counts)
    assert (counts % 32 != 0).any()        # ragged group tails exercised
    nbt = int(sum(-(-int(c) // 32) for c in counts))
    y = torch.empty(x.shape, dtype=torch.bfloat16, device="cuda")
    m = torch.empty((M.grouped_mask_rows_max(rows, 32, G), cols), dtype=torch.int32, device="cuda")
    m.view(torch.uint8).fill_(FILL)
    s = torch.full((M.grouped_scale_rows_max(rows, 32, G), cols), FILL, dtype=torch.uint8,
                   device="cuda")
    xd, gl = dev(x), dev(counts)
    M.mxfp4_grouped_qdq(xd, gl, y, m, s)
    # the GROUPED-layout STE of an upstream gradient (the same tokens reused)
    gi = torch.empty_like(xd)
    M.mxfp4_ste_bwd(xd, m, gi, layout=M.GROUPED, group_list=gl)
    torch.cuda.synchronize()
    yo, co, eo = oracle.grouped_cols(x, counts, 32)
    _eq(host(y), yo, "y")
    mw = host(m)
    bits, clean = unpack_grouped_bitmap(mw[:nbt], rows, counts, 32)
    _eq(bits, co, "grouped bitmap")
    assert clean
    assert (mw[nbt:].view(np.uint8) == FILL).all()
    sh = host(s)
    _eq(sh[:nbt], eo, "scales")
    assert (sh[nbt:] == FILL).all()
    _eq(host(gi), oracle.ste_bwd(x, co), "grouped STE")


def test_moe_grouped_kmajor_full(oracle):
    x, counts = W.moe_grouped()
    rows, cols = x.shape
    kb = M.kmajor_k_blocks(rows, 32, len(counts))
    codes = torch.full((cols, kb * 16), FILL, dtype=torch.uint8, device="cuda")
    sc = torch.full((cols, kb), FILL, dtype=torch.uint8, device="cuda")
    M.mxfp4_quant_pack_kmajor(dev(x), codes, sc, group_list=dev(counts))
    torch.cuda.synchronize()
    co, so, nbt = oracle.pack_kmajor(x, 32, group_list=counts, k_blocks=kb, fill=FILL)
    assert nbt <= kb
    _eq(host(codes), co, "codes_t")
    _eq(host(sc), so, "scales_t")


@pytest.mark.parametrize("block", [32, 128])
def test_weight_pack_full(oracle, block):
    x = W.weight_pack()
    rows, cols = x.shape
    xd = dev(x)
    codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device="cuda")
    sc = torch.empty((rows, cols // block), dtype=torch.uint8, device="cuda")
    M.mxfp4_quant_pack(xd, codes, sc, block=block)
    torch.cuda.synchronize()
    co, so = oracle.pack_rows(x, block)
    _eq(host(codes), co, "codes")
    _eq(host(sc), so, "scales")
    del co, so
    # dequantizing the packed form (on the GPU) equals the QDQ output
    y = torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda")
    M.mxfp4_dequant(codes, sc, y, block=block)
    del codes, sc
    yq = torch.empty_like(y)
    M.mxfp4_qdq_fwd(xd, M.ROW, y_row=yq, block=block)
    torch.cuda.synchronize()
    yo, _, _ = oracle.qdq_rows(x, block)
    _eq(host(y), yo, "decode(pack)")
    _eq(host(yq), yo, "qdq")


def test_weight_pack_kmajor_full(oracle):
    x = W.weight_pack()
    rows, cols = x.shape
    kb = M.kmajor_k_blocks(rows, 32)
    codes = torch.empty((cols, kb * 16), dtype=torch.uint8, device="cuda")
    sc = torch.empty((cols, kb), dtype=torch.uint8, device="cuda")
    M.mxfp4_quant_pack_kmajor(dev(x), codes, sc)
    torch.cuda.synchronize()
    co, so, _ = oracle.pack_kmajor(x, 32, k_blocks=kb)
    _eq(host(codes), co, "codes_t")
    _eq(host(sc), so, "scales_t")


def test_moe_mxfp8_rows_full(oracle):
    """MXFP8 (E4M3) of a grad_output-sized bf16 tensor, 32768 x 7168."""
    x, _ = W.moe_grouped()
    rows, cols = x.shape
    q = torch.empty((rows, cols), dtype=torch.uint8, device="cuda")
    s = torch.empty((rows, cols // 32), dtype=torch.uint8, device="cuda")
    M.mxfp8_quant(dev(x), q, s)
    torch.cuda.synchronize()
    qo, so = oracle.mxfp8_rows(x)
    _eq(host(q), qo, "q")
    _eq(host(s), so, "scales")


def test_moe_mxfp8_kmajor_full(oracle):
    """Grouped K-major MXFP8 of the MoE tokens (the TN operand), 8 experts."""
    x, counts = W.moe_grouped()
    rows, cols = x.shape
    kb = M.mxfp8_kmajor_k_blocks(rows, len(counts))
    q = torch.full((cols, kb * 32), FILL, dtype=torch.uint8, device="cuda")
    s = torch.full((cols, kb), FILL, dtype=torch.uint8, device="cuda")
    M.mxfp8_quant_kmajor(dev(x), q, s, group_list=dev(counts))
    torch.cuda.synchronize()
    qo, so, nbt = oracle.mxfp8_kmajor(x, "e4m3", counts, 1, k_blocks=kb, fill=FILL)
    _eq(host(q), qo, "q_t")
    _eq(host(s), so, "scales_t")
