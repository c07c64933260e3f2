"""GPU parity of the K-major packed operand (column-wise and grouped blocks
stored packed with the reduction dimension contiguous) and of the decode
kernel, through the C-ABI binding, bit for bit against the oracle.  Output
buffers are prefilled with a marker byte, which must survive past the
block-rows the blocking produces, and carry a canary past their end."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import Guarded, dev, host

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


def make_x(shape, dtype, seed):
    g = np.random.default_rng(seed)
    a = (g.standard_t(3, size=shape) * np.exp2(g.uniform(-8, 8, (1, shape[1])))).astype(np.float32)
    a.reshape(-1)[::97] = 0.0
    a.reshape(-1)[5::113] = -0.0
    return W.f32_to_bf16_bits(a) if dtype == "bf16" else a


def run_kmajor(x, block, rule, kb, counts=None, list_type=1, raw_list=False):
    rows, cols = x.shape
    codes = Guarded((cols, kb * block // 2), torch.uint8, fill=FILL)
    sc = Guarded((cols, kb), torch.uint8, fill=FILL)
    gl = None
    if counts is not None:
        gl = dev(np.asarray(counts if list_type == 1 or raw_list else np.cumsum(counts), np.int64))
    M.mxfp4_quant_pack_kmajor(dev(x), codes.t, sc.t, block=block, rule=rule, group_list=gl,
                              group_list_type=list_type)
    torch.cuda.synchronize()
    codes.check_tail()
    sc.check_tail()
    return host(codes.t), host(sc.t)


# ------------------------------------------------------------------ dense

# rows span several 256-row tiles and ragged block tails; cols span several
# 64-column tiles, partial tiles, and widths that are not multiples of 8
DENSE_SHAPES = [(1, 1), (37, 8), (256, 64), (300, 72), (513, 129), (1000, 136), (64, 200),
                (129, 7), (700, 520)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("block", [32, 128])
@pytest.mark.parametrize("rule", ["floor", "amct"])
@pytest.mark.parametrize("shape", DENSE_SHAPES)
def test_kmajor_dense(oracle, dtype, block, rule, shape):
    x = make_x(shape, dtype, seed=shape[0] + shape[1])
    # minimal k_blocks, minimal + spare blocks, and the aligned default
    kb = (M.kmajor_k_blocks(shape[0], block, align=False) + 3 if shape[1] % 2 else
          M.kmajor_k_blocks(shape[0], block, align=shape[0] % 2 == 0))
    c, s = run_kmajor(x, block, rule, kb)
    co, so, _ = oracle.pack_kmajor(x, block, rule, k_blocks=kb, fill=FILL)
    assert np.array_equal(c, co)
    assert np.array_equal(s, so)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rule", ["floor", "amct"])
@pytest.mark.parametrize("block", [32, 128])
def test_kmajor_edge_blocks(oracle, dtype, rule, block):
    """Ties, codebook points, clipped maxima, signed zeros and tiny / subnormal
    scales (the generic snap for FLOOR), one planted block per column."""
    e = W.edge_blocks_f32(32)
    if block == 128:
        e = e[: (e.shape[0] // 4) * 4].reshape(-1, 128)
    x32 = np.ascontiguousarray(np.concatenate([e.T, e.T[::-1]], axis=0))   # [2*block, n_blocks]
    x = W.f32_to_bf16_bits(x32) if dtype == "bf16" else x32
    kb = M.kmajor_k_blocks(x.shape[0], block)
    c, s = run_kmajor(x, block, rule, kb)
    co, so, _ = oracle.pack_kmajor(x, block, rule, k_blocks=kb, fill=FILL)
    assert np.array_equal(c, co)
    assert np.array_equal(s, so)


def tiny_scale_blocks(block):
    """bf16 columns of `block` rows, each one FLOOR block whose max lies below
    2^-122 (E8M0 byte 0, 1 or 2: the generic snap): for each of a set of such
    maxima, every bf16 magnitude up to it with both signs, the max itself at
    a varying row.  Returns bf16 bits [block, n_blocks]."""
    blocks = []
    for amax in (0x0001, 0x0003, 0x0040, 0x007F, 0x0080, 0x00C0, 0x00FF, 0x0100, 0x0155, 0x01FF,
                 0x0200, 0x0250, 0x027F):
        mags = np.arange(0, amax + 1, dtype=np.uint16)
        vals = np.concatenate([mags, mags | np.uint16(0x8000)])
        per = block - 1
        for i in range(0, len(vals), per):
            chunk = list(vals[i:i + per])
            top = amax if (i // per) % 2 == 0 else amax | 0x8000
            chunk.insert(min((i // per) % block, len(chunk)), top)
            b = np.zeros(block, np.uint16)
            b[:len(chunk)] = chunk
            blocks.append(b)
    return np.ascontiguousarray(np.stack(blocks, axis=1))


@pytest.mark.parametrize("block", [32, 128])
def test_kmajor_tiny_scales_every_value(oracle, block):
    """Every bf16 magnitude (both signs) under FLOOR block maxima below 2^-122,
    i.e. E8M0 bytes 0-2, where the kernel takes its generic snap."""
    x = tiny_scale_blocks(block)
    rows, cols = x.shape
    kb = M.kmajor_k_blocks(rows, block)
    c, s = run_kmajor(x, block, "floor", kb)
    co, so, _ = oracle.pack_kmajor(x, block, "floor", k_blocks=kb, fill=FILL)
    assert np.array_equal(c, co)
    assert np.array_equal(s, so)
    assert (so[:, 0] <= 2).all() and cols > 60


# ------------------------------------------------------------------ grouped

GROUP_CASES = [
    (700, 24, [100, 0, 37, 300, 1, 262]),
    (512, 136, [64, 64, 128, 0, 256]),
    (97, 40, [0, 97]),
    (1000, 520, None),
    (33, 8, [33]),
    (300, 66, [0, 0, 300, 0]),
    (1500, 40, 40),     # 40 groups: decoded by the wave scan
    (3000, 24, 100),    # 100 groups: two 64-group scan steps
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("block", [32, 128])
@pytest.mark.parametrize("rule", ["floor", "amct"])
@pytest.mark.parametrize("case", range(len(GROUP_CASES)))
@pytest.mark.parametrize("list_type", [1, 0])
def test_kmajor_grouped(oracle, dtype, block, rule, case, list_type):
    rows, cols, counts = GROUP_CASES[case]
    if counts is None or isinstance(counts, int):
        counts = W.ragged_counts(rows, counts or 9, seed=case, zero_groups=2 if counts is None else 7)
    counts = np.asarray(counts, np.int64)
    x = make_x((rows, cols), dtype, seed=case + 70)
    kb = M.kmajor_k_blocks(rows, block, len(counts), align=case % 2 == 0) + case % 3 // 2
    c, s = run_kmajor(x, block, rule, kb, counts, list_type)
    co, so, nbt = oracle.pack_kmajor(x, block, rule, group_list=counts, k_blocks=kb, fill=FILL)
    assert np.array_equal(c, co)
    assert np.array_equal(s, so)
    assert (c[:, nbt * block // 2:] == FILL).all()          # block-rows past NBT untouched


@pytest.mark.parametrize("list_type,gl", [(1, [100, -5, 50, 400]), (0, [100, 50, 250, 400]),
                                          (0, [-7, 33, 20, 300])])
@pytest.mark.parametrize("block", [32, 128])
def test_kmajor_inconsistent_list_is_clamped(oracle, list_type, gl, block):
    """An inconsistent group list is clamped (negative counts are 0, ends into
    [previous end, rows]); the operand equals the oracle's for the clamped list."""
    from test_gpu_parity import clamp_group_list
    rows, cols = 300, 72
    x = make_x((rows, cols), "bf16", 13)
    counts = clamp_group_list(gl, rows, list_type)
    kb = M.kmajor_k_blocks(rows, block, len(gl))
    c, s = run_kmajor(x, block, "floor", kb, np.asarray(gl, np.int64), list_type=list_type,
                      raw_list=True)
    co, so, _ = oracle.pack_kmajor(x, block, "floor", group_list=counts, k_blocks=kb, fill=FILL)
    assert np.array_equal(c, co)
    assert np.array_equal(s, so)


def test_kmajor_decodes_to_column_qdq(oracle):
    """GPU pack then GPU decode of the K-major operand gives the column-wise
    QDQ values transposed, zeros at the padding of the short last block."""
    x = make_x((300, 72), "bf16", 3)
    kb = M.kmajor_k_blocks(300, 32)
    codes = torch.empty((72, kb * 16), dtype=torch.uint8, device="cuda")
    sc = torch.empty((72, kb), dtype=torch.uint8, device="cuda")
    M.mxfp4_quant_pack_kmajor(dev(x), codes, sc)
    y = torch.empty((72, kb * 32), dtype=torch.bfloat16, device="cuda")
    M.mxfp4_dequant(codes, sc, y)
    torch.cuda.synchronize()
    yo, _, _ = oracle.qdq_cols(x, 32)
    yh = host(y)
    assert np.array_equal(yh[:, :300], yo.T)
    assert (yh[:, 300:320] == 0).all()       # padding of the short last block (block-rows past it untouched)


# ------------------------------------------------------------------ decode

DQ_SHAPES = [(1, 1), (3, 7), (5, 64), (17, 96), (9, 256), (33, 1000), (64, 4096), (7, 8200),
             (130, 384)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("block", [32, 128])
@pytest.mark.parametrize("shape", DQ_SHAPES)
def test_dequant_random_bytes(oracle, dtype, block, shape):
    """Random code bytes and random E8M0 bytes (all 256 values occur, so the
    subnormal and overflow-to-inf cases are exercised), flat and per-row
    launches, ragged and odd widths."""
    rows, cols = shape
    g = np.random.default_rng(rows * 131 + cols)
    codes = g.integers(0, 256, (rows, (cols + 1) // 2), dtype=np.uint8)
    nb = -(-cols // block)
    sc = g.integers(0, 256, (rows, nb), dtype=np.uint8)
    sc.reshape(-1)[: min(256, sc.size)] = np.arange(min(256, sc.size), dtype=np.uint8)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    y = Guarded((rows, cols), tdt)
    M.mxfp4_dequant(dev(codes), dev(sc), y.t, block=block)
    torch.cuda.synchronize()
    want = oracle.unpack_rows(codes, sc, cols, block, np.uint16 if dtype == "bf16" else np.float32)
    got = host(y.t)
    if dtype == "f32":
        got, want = got.view(np.uint32), want.view(np.uint32)
    assert np.array_equal(got, want)
    y.check_tail()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_dequant_every_nibble_and_byte(oracle, dtype):
    """All 16 nibbles under all 256 scale bytes, one 32-block per row."""
    nib = np.arange(16, dtype=np.uint8)
    codes = np.tile((nib[0::2] | (nib[1::2] << 4))[None, :], (256, 2))     # 16 bytes = 32 values
    sc = np.arange(256, dtype=np.uint8)[:, None]
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    y = torch.empty((256, 32), dtype=tdt, device="cuda")
    M.mxfp4_dequant(dev(np.ascontiguousarray(codes)), dev(sc), y, block=32)
    torch.cuda.synchronize()
    want = oracle.unpack_rows(codes, sc, 32, 32, np.uint16 if dtype == "bf16" else np.float32)
    got = host(y)
    if dtype == "f32":
        got, want = got.view(np.uint32), want.view(np.uint32)
    assert np.array_equal(got, want)


