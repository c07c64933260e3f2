"""GPU parity of the MXFP8 (OCP MX) quantization of grad_output, through the
C-ABI binding, bit for bit against the oracle: every bf16 value under several
block maxima, exact fp32 midpoints (ties to even), zero / subnormal /
saturating blocks, ragged widths (flat, row-vector and scalar launches), and
a full-size tensor on sampled rows.  Outputs carry a canary past their end."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import Guarded, dev, host

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


def run(x, fmt):
    rows, cols = x.shape
    q = Guarded((rows, cols), torch.uint8)
    s = Guarded((rows, -(-cols // 32)), torch.uint8)
    M.mxfp8_quant(dev(x), q.t, s.t, fmt=fmt)
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
def test_mxfp8_shapes(oracle, dtype, fmt, shape):
    g = np.random.default_rng(shape[0] * 7 + shape[1])
    a = (g.standard_t(3, size=shape) * np.exp2(g.uniform(-40, 40, (shape[0], 1)))).astype(np.float32)
    a.reshape(-1)[::53] = 0.0
    a.reshape(-1)[7::61] = -0.0
    if shape[0] > 2:
        a[1] = 2.0 ** -140                   # fp32 subnormal block maxima
        a[2] = 0.0                           # all-zero row
    x = W.f32_to_bf16_bits(a) if dtype == "bf16" else a
    q, s = run(x, fmt)
    qo, so = oracle.mxfp8_rows(x, fmt)
    assert np.array_equal(s, so)
    assert np.array_equal(q, qo)


def test_mxfp8_edge_blocks(oracle):
    """The planted edge blocks of the MXFP4 tests (ties, clipped maxima, signed
    zeros, tiny and subnormal scales) as MXFP8 input."""
    e = W.edge_blocks_f32(32)
    for x in (e, W.f32_to_bf16_bits(e)):
        for fmt in ("e4m3", "e5m2"):
            q, s = run(np.ascontiguousarray(x), fmt)
            qo, so = oracle.mxfp8_rows(np.ascontiguousarray(x), fmt)
            assert np.array_equal(s, so) and np.array_equal(q, qo)


def test_mxfp8_grad_output_sampled(oracle):
    """A grad_output-sized bf16 tensor (32768 x 7168, N(0,1) tokens of the MoE
    layer): sampled rows against the oracle."""
    x, _ = W.moe_grouped()
    rows, cols = x.shape
    q = torch.empty((rows, cols), dtype=torch.uint8, device="cuda")
    s = torch.empty((rows, cols // 32), dtype=torch.uint8, device="cuda")
    M.mxfp8_quant(dev(x), q, s)
    torch.cuda.synchronize()
    ri = np.sort(np.random.default_rng(9).choice(rows, 512, replace=False))
    rit = torch.from_numpy(ri).cuda()
    qo, so = oracle.mxfp8_rows(x[ri])
    assert np.array_equal(host(q[rit]), qo)
    assert np.array_equal(host(s[rit]), so)
