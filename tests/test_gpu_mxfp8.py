"""GPU parity of the MXFP8 (OCP MX) quantization of grad_output, through the
C-ABI binding, bit for bit against the oracle: every bf16 value under several
block maxima, exact fp32 midpoints (ties to even), zero / subnormal /
saturating blocks, ragged widths (flat, row-vector and scalar launches); the
full-size MoE tensors are in test_gpu_full_size.py.  Outputs carry a canary
past their end."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import Guarded, dev, host
from mx_tolerance import mx_matmul_bound

pytestmark = pytest.mark.gpu

M = None


@pytest.fixture(scope="module", autouse=True)
def lib():
    global M
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mxfp4_fake_quantization_amd as mod
    mod._load()
    M = mod
    yield


def run(x, fmt, block=32):
    rows, cols = x.shape
    q = Guarded((rows, cols), torch.uint8)
    s = Guarded((rows, -(-cols // block)), torch.uint8)
    M.mxfp8_quant(dev(x), q.t, s.t, fmt=fmt, block=block)
    torch.cuda.synchronize()
    q.check_tail()
    s.check_tail()
    return host(q.t), host(s.t)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("j", [0, -5, 20, -118, 100])
def test_mxfp8_every_bf16_value(oracle, fmt, j):
    M_ = np.float32(1.5 * 2.0 ** j)
    allb = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    v = W.bf16_bits_to_f32(allb)
    v = v[np.isfinite(v) & (np.abs(v) <= M_)]
    n = -(-v.size // 31) * 31
    vv = np.zeros(n, np.float32)
    vv[: v.size] = v
    x = W.f32_to_bf16_bits(np.concatenate([np.full((n // 31, 1), M_, np.float32), vv.reshape(-1, 31)], axis=1))
    q, s = run(x, fmt)
    qo, so = oracle.mxfp8_rows(x, fmt)
    assert np.array_equal(s, so)
    assert np.array_equal(q, qo)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_mxfp8_fp32_midpoints_tie_to_even(oracle, fmt):
    """fp32 elements exactly on the midpoint between neighbouring fp8 values
    (and one ulp either side), in every binade, under a block maximum of
    1.0 * 2^j."""
    mb, bias, emax = (3, 7, 8) if fmt == "e4m3" else (2, 15, 15)
    vals = []
    for e in range(1 - bias - mb, emax + 1):
        step = 2.0 ** max(e - mb, 1 - bias - mb)
        for m in range(1 << mb):
            base = 2.0 ** e * (1 + m / (1 << mb)) if e >= 1 - bias else m * step
            mid = base + step / 2
            for t in (mid, np.nextafter(np.float32(mid), np.float32(0)), np.nextafter(np.float32(mid), np.float32(np.inf))):
                vals.append(t)
    vals = np.asarray(vals, np.float64)
    vals = vals[vals < 2.0 ** emax]
    rows = []
    for j in (0, -40, 60):
        sc = 2.0 ** (j - emax)
        v = (vals * sc).astype(np.float32)
        v = np.concatenate([v, -v])
        n = -(-v.size // 31) * 31
        vv = np.zeros(n, np.float32)
        vv[: v.size] = v
        rows.append(np.concatenate([np.full((n // 31, 1), np.float32(2.0 ** j), np.float32), vv.reshape(-1, 31)], axis=1))
    x = np.ascontiguousarray(np.concatenate(rows))
    q, s = run(x, fmt)
    qo, so = oracle.mxfp8_rows(x, fmt)
    assert np.array_equal(s, so)
    assert np.array_equal(q, qo)


SHAPES = [(1, 1), (3, 7), (5, 32), (9, 77), (17, 200), (33, 96), (64, 4096), (130, 384), (7, 1000)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("block", [32, 128])
def test_mxfp8_shapes(oracle, dtype, fmt, shape, block):
    g = np.random.default_rng(shape[0] * 7 + shape[1])
    a = (g.standard_t(3, size=shape) * np.exp2(g.uniform(-40, 40, (shape[0], 1)))).astype(np.float32)
    a.reshape(-1)[::53] = 0.0
    a.reshape(-1)[7::61] = -0.0
    if shape[0] > 2:
        a[1] = 2.0 ** -140                   # fp32 subnormal block maxima
        a[2] = 0.0                           # all-zero row
    x = W.f32_to_bf16_bits(a) if dtype == "bf16" else a
    q, s = run(x, fmt, block)
    qo, so = oracle.mxfp8_rows(x, fmt, block)
    assert np.array_equal(s, so)
    assert np.array_equal(q, qo)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_mxfp8_block128_every_bf16_value(oracle, fmt):
    """Every finite bf16 value in blocks of 128 whose maximum sits in any of
    the four 32-element quarters (the block-128 maximum spans 16 lanes)."""
    allb = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    v = W.bf16_bits_to_f32(allb)
    v = v[np.isfinite(v) & (np.abs(v) <= 2.0 ** 20)]
    n = -(-v.size // 127) * 127
    vv = np.zeros(n, np.float32)
    vv[: v.size] = v
    body = vv.reshape(-1, 127)
    x = np.zeros((body.shape[0], 128), np.float32)
    pos = 32 * (np.arange(body.shape[0]) % 4) + 7
    for r in range(body.shape[0]):
        x[r] = np.insert(body[r], pos[r], np.float32(1.5 * 2.0 ** 20))
    xb = W.f32_to_bf16_bits(x)
    q, s = run(xb, fmt, 128)
    qo, so = oracle.mxfp8_rows(xb, fmt, 128)
    assert np.array_equal(s, so) and np.array_equal(q, qo)


def test_mxfp8_edge_blocks(oracle):
    """The planted edge blocks of the MXFP4 tests (ties, clipped maxima, signed
    zeros, tiny and subnormal scales) as MXFP8 input."""
    e = W.edge_blocks_f32(32)
    for x in (e, W.f32_to_bf16_bits(e)):
        for fmt in ("e4m3", "e5m2"):
            q, s = run(np.ascontiguousarray(x), fmt)
            qo, so = oracle.mxfp8_rows(np.ascontiguousarray(x), fmt)
            assert np.array_equal(s, so) and np.array_equal(q, qo)



# ---- K-major MXFP8 (grouped column-wise operand of the TN product) ------------------

def run_kmajor(x, fmt, group_list=None, list_type=1, k_blocks=None, dev_list=False):
    rows, cols = x.shape
    if k_blocks is None:
        k_blocks = M.mxfp8_kmajor_k_blocks(rows, None if group_list is None else len(group_list))
    q = Guarded((cols, k_blocks * 32), torch.uint8)
    s = Guarded((cols, k_blocks), torch.uint8)
    gl = group_list
    if gl is not None and dev_list:
        gl = torch.tensor(list(gl), dtype=torch.int64, device="cuda")
    M.mxfp8_quant_kmajor(dev(x), q.t, s.t, fmt=fmt, group_list=gl, group_list_type=list_type)
    torch.cuda.synchronize()
    q.check_tail()
    s.check_tail()
    return host(q.t), host(s.t), k_blocks


KM_SHAPES = [(1, 1), (31, 7), (32, 64), (100, 130), (257, 64), (64, 1000), (300, 72)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("shape", KM_SHAPES)
def test_mxfp8_kmajor_dense(oracle, dtype, fmt, shape):
    g = np.random.default_rng(shape[0] * 13 + shape[1])
    a = (g.standard_t(3, size=shape) * np.exp2(g.uniform(-30, 30, (1, shape[1])))).astype(np.float32)
    a.reshape(-1)[::37] = 0.0
    a.reshape(-1)[5::41] = -0.0
    x = W.f32_to_bf16_bits(a) if dtype == "bf16" else a
    q, s, kb = run_kmajor(x, fmt)
    qo, so, nbt = oracle.mxfp8_kmajor(x, fmt, k_blocks=kb, fill=0xA5)
    assert np.array_equal(q[:, :32 * nbt], qo[:, :32 * nbt])
    assert np.array_equal(s[:, :nbt], so[:, :nbt])
    assert (q[:, 32 * nbt:] == 0xA5).all() and (s[:, nbt:] == 0xA5).all()   # untouched


GROUPED = [([45, 0, 1, 64, 30], 1), (list(np.cumsum([45, 0, 1, 64, 30])), 0), ("forty", 1)]


@pytest.mark.parametrize("gl,lt", GROUPED, ids=["counts", "ends", "forty"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_mxfp8_kmajor_grouped(oracle, gl, lt, dtype):
    rows, cols = 140, 96
    if gl == "forty":
        rows = 700
        gl = W.ragged_counts(rows, 40, seed=5, zero_groups=6).tolist()
    g = np.random.default_rng(len(gl) + rows)
    a = g.standard_normal((rows, cols)).astype(np.float32)
    x = W.f32_to_bf16_bits(a) if dtype == "bf16" else a
    q, s, kb = run_kmajor(x, "e4m3", gl, lt)
    qo, so, nbt = oracle.mxfp8_kmajor(x, "e4m3", gl, lt, k_blocks=kb, fill=0xA5)
    assert np.array_equal(q, qo) and np.array_equal(s, so)


@pytest.mark.parametrize("list_type,gl", [(1, [100, -5, 50, 400]), (0, [100, 50, 250, 400]), (0, [-7, 33, 20, 300])])
def test_mxfp8_kmajor_inconsistent_list_is_clamped(oracle, list_type, gl):
    """A device list with negative counts, ends past rows or decreasing ends is
    clamped into range (the documented treatment), block-rows as the oracle's
    of the clamped counts."""
    from test_gpu_parity import clamp_group_list
    rows, cols = 300, 72
    x = W.f32_to_bf16_bits(np.random.default_rng(4).standard_normal((rows, cols)).astype(np.float32))
    q, s, kb = run_kmajor(x, "e4m3", gl, list_type, dev_list=True)
    counts = clamp_group_list(gl, rows, list_type)
    qo, so, nbt = oracle.mxfp8_kmajor(np.ascontiguousarray(x[:int(counts.sum())]), "e4m3", counts, 1,
                                      k_blocks=kb, fill=0xA5)
    assert np.array_equal(q, qo) and np.array_equal(s, so)



def test_tn_weight_gradient_end_to_end(oracle):
    """TN: x and grad_output quantized on the GPU into K-major grouped MXFP8,
    then the K-split grouped matmul gives each expert's dW = x_g^T dy_g; the
    operands bit-exact against the oracle's, the products against the oracle's
    exact sums within the matrix-core bound (mx_tolerance)."""
    g = np.random.default_rng(17)
    counts = [70, 0, 33, 97]
    T, Kin, N = sum(counts), 96, 80
    x = W.f32_to_bf16_bits(g.standard_normal((T, Kin)).astype(np.float32))
    dy = W.f32_to_bf16_bits(g.standard_normal((T, N)).astype(np.float32))
    kb = M.mxfp8_kmajor_k_blocks(T, len(counts))
    qa = torch.empty((Kin, kb * 32), dtype=torch.uint8, device="cuda")
    sa = torch.empty((Kin, kb), dtype=torch.uint8, device="cuda")
    qb = torch.empty((N, kb * 32), dtype=torch.uint8, device="cuda")
    sb = torch.empty((N, kb), dtype=torch.uint8, device="cuda")
    M.mxfp8_quant_kmajor(dev(x), qa, sa, group_list=counts)
    M.mxfp8_quant_kmajor(dev(dy), qb, sb, group_list=counts)
    c = torch.empty((len(counts), Kin, N), dtype=torch.float32, device="cuda")
    M.mxfp4_grouped_matmul(qa, sa, qb, sb, c, K=T, group_list=counts, group_type=M.GROUP_K, b_fmt="e4m3",
                           k_blocks=kb)
    torch.cuda.synchronize()
    qao, sao, nbt = oracle.mxfp8_kmajor(x, "e4m3", counts, 1, k_blocks=kb, fill=0)
    qbo, sbo, _ = oracle.mxfp8_kmajor(dy, "e4m3", counts, 1, k_blocks=kb, fill=0)
    # the operands themselves are bit-exact
    assert np.array_equal(host(qa)[:, :32 * nbt], qao[:, :32 * nbt])
    assert np.array_equal(host(qb)[:, :32 * nbt], qbo[:, :32 * nbt])
    assert np.array_equal(host(sa)[:, :nbt], sao[:, :nbt]) and np.array_equal(host(sb)[:, :nbt], sbo[:, :nbt])
    sao[:, nbt:] = 127
    sbo[:, nbt:] = 127
    A = oracle.mxfp8_decode(qao, sao, "e4m3", np.float64)
    B = oracle.mxfp8_decode(qbo, sbo, "e4m3", np.float64)
    padded = [32 * (-(-cc // 32)) for cc in counts]
    exp = oracle.grouped_matmul(A, np.ascontiguousarray(B.T), padded, oracle.GROUP_K, 1)
    got = host(c).astype(np.float64)
    k0 = 0
    for gi, pc in enumerate(padded):
        if pc:
            bound = mx_matmul_bound(A[:, k0:k0 + pc], B[:, k0:k0 + pc]) + 1e-30
            ratio = np.abs(got[gi] - exp[gi]) / bound
            w = np.unravel_index(ratio.argmax(), ratio.shape)
            assert (ratio <= 1).all(), f"group {gi}: worst error / bound {ratio.max():.3g} at {w}"
        k0 += pc
    assert (got[1] == 0).all()   # the empty expert
