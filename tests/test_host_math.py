"""CPU check of the kernels' integer MXFP4 math (csrc/mxfp4_math.h) against the
oracle, before any GPU run: a host build of the same functions, driven the way
a kernel lane drives them, must agree bit for bit with the oracle on every
bf16 magnitude under many block maxima (normal and subnormal), on heavy-tailed
fp32 data, and for both scale rules."""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mxfp4_fake_quantization_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "host_math_check.cpp")
CLANG = "/opt/rocm/llvm/bin/clang++"


@pytest.fixture(scope="module")
def host(tmp_path_factory):
    if not os.path.exists(CLANG):
        pytest.skip("ROCm clang++ not available")
    out = tmp_path_factory.mktemp("hostmath") / "libhostmath.so"
    subprocess.run([CLANG, "-O2", "-std=c++17", "-shared", "-fPIC", "-I", CSRC, SRC, "-o", str(out)],
                   check=True)
    lib = ctypes.CDLL(str(out))
    vp = ctypes.c_void_p
    lib.host_qdq_rows.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_float, vp, vp, vp, vp, vp]
    return lib


def run_host(lib, x, block, rule, sf=6.0):
    rows, cols = x.shape
    y = np.empty_like(x)
    clip = np.empty((rows, cols), np.uint8)
    e8 = np.empty((rows, -(-cols // block)), np.uint8)
    nib = np.empty((rows, cols), np.uint8)
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    dt = 1 if x.dtype == np.uint16 else 0
    lib.host_qdq_rows(dt, rows, cols, block, 0 if rule == "floor" else 1, sf, p(x), p(y), p(clip),
                      p(e8), p(nib))
    return y, clip.astype(bool), e8, nib


def pack_nibbles(nib):
    rows, cols = nib.shape
    if cols % 2:
        nib = np.concatenate([nib, np.zeros((rows, 1), np.uint8)], axis=1)
    return (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)


def compare(lib, oracle, x, block, rule, sf=6.0):
    y, clip, e8, nib = run_host(lib, x, block, rule, sf)
    yo, co, eo = oracle.qdq_rows(x, block, rule, sf)
    codes, sc = oracle.pack_rows(x, block, rule, sf)
    bad = np.argwhere(y != yo)
    assert bad.size == 0, f"y mismatch at {bad[:5]}: x={x[tuple(bad[0])]:#x} host={y[tuple(bad[0])]:#x} oracle={yo[tuple(bad[0])]:#x}"
    assert np.array_equal(clip, co)
    assert np.array_equal(e8, eo)
    assert np.array_equal(pack_nibbles(nib), codes)


def bf16_blocks_under_max(max_bits, per=31):
    """Blocks [M, v...] covering every bf16 magnitude v <= M, both signs."""
    allb = np.arange(0, 0x7F80, dtype=np.uint16)
    v = allb[allb <= max_bits]
    vals = np.concatenate([v, v | np.uint16(0x8000)])
    n = len(vals)
    nrows = -(-n // per)
    flat = np.zeros(nrows * per, np.uint16)
    flat[:n] = vals
    out = np.empty((nrows, per + 1), np.uint16)
    out[:, 0] = max_bits
    out[:, 1:] = flat.reshape(nrows, per)
    return out


@pytest.mark.parametrize("rule", ["floor", "amct"])
def test_every_bf16_magnitude_under_many_maxima(host, oracle, rule):
    maxima = set()
    for e in list(range(0, 8)) + [20, 97, 98, 120, 124, 127, 130, 200, 250, 252, 253, 254]:
        for m in (0, 1, 31, 32, 33, 63, 64, 95, 96, 97, 127):
            maxima.add((e << 7) | m)
    for mx in sorted(maxima):
        if mx == 0 or mx >= 0x7F80:
            continue
        x = bf16_blocks_under_max(mx)
        compare(host, oracle, x, 32, rule)


@pytest.mark.parametrize("rule", ["floor", "amct"])
@pytest.mark.parametrize("block", [32, 128])
def test_bf16_workload_like_and_edges(host, oracle, rule, block):
    x, _, _ = W.weight_4k(seed=2, rows=256, cols=1024, with_grad=False)
    compare(host, oracle, x, block, rule)
    e = W.f32_to_bf16_bits(W.edge_blocks_f32(32))
    compare(host, oracle, e, 32, rule)
    compare(host, oracle, np.ascontiguousarray(e.T), block, rule)


@pytest.mark.parametrize("rule", ["floor", "amct"])
@pytest.mark.parametrize("sf", [6.0, 4.0, 7.3])
def test_fp32_heavy_tailed_all_scales(host, oracle, rule, sf):
    if rule == "floor" and sf != 6.0:
        pytest.skip("scale_factor only matters for amct")
    g = np.random.default_rng(7)
    rows = 3000
    x = (g.standard_t(2.5, size=(rows, 96)) *
         np.exp2(g.uniform(-149, 120, (rows, 1)))).astype(np.float32)
    x[::7, 5] = -0.0
    x[::11, :32] = 0.0
    compare(host, oracle, x, 32, rule, sf)
    compare(host, oracle, x[:, :80].copy(), 32, rule, sf)   # ragged rows


def test_fp32_exhaustive_mantissa_sweep(host, oracle):
    """All fp32 mantissas at a few exponents (relative to a fixed block max),
    covering every tie and neighbour in the 1..6 code range."""
    g = np.random.default_rng(9)
    for k in (-127, -126, -125, -124, -30, 0, 100):
        scale = np.float64(2.0) ** k
        ties = np.array([0, 1, (1 << 23) - 1] + [m + d for m in (0x200000, 0x400000, 0x600000)
                                                 for d in (-1, 0, 1)], np.uint32)
        mant = np.concatenate([np.arange(0, 1 << 23, 97, dtype=np.uint32), ties])
        for e in (-3, -2, -1, 0, 1, 2):
            v = ((np.uint32(127 + e) << np.uint32(23)) | mant).view(np.float32).astype(np.float64) * scale
            v = v[v <= 6 * scale].astype(np.float32)
            per = 31
            n = len(v) - len(v) % per
            blocks = np.empty((n // per, 32), np.float32)
            blocks[:, 0] = np.float32(6 * scale)
            blocks[:, 1:] = (v[:n] * np.where(g.random(n) < 0.5, -1, 1).astype(np.float32)).reshape(-1, per)
            compare(host, oracle, blocks, 32, "floor")
            if k >= -30:
                compare(host, oracle, blocks, 32, "amct")


def test_packed_column_params_match_scalar_rule(host):
    host.host_check_packed_params.restype = ctypes.c_int
    assert host.host_check_packed_params() == 0


def test_generic_decode_every_nibble_and_byte(host, oracle):
    """The kernels' generic decode (every E8M0 byte, every nibble) equals the
    oracle's unpack in bf16 and fp32."""
    out = np.empty(256 * 16, np.uint16)
    out32 = np.empty(256 * 16, np.uint32)
    host.host_decode_all(out.ctypes.data_as(ctypes.c_void_p), out32.ctypes.data_as(ctypes.c_void_p))
    nib = np.arange(16, dtype=np.uint8)
    codes = np.repeat((nib[0::2] | (nib[1::2] << 4))[None, :], 256, axis=0)   # 8 bytes = 16 nibbles
    scales = np.arange(256, dtype=np.uint8)[:, None]
    want16 = oracle.unpack_rows(codes, scales, 16, 32, np.uint16)
    want32 = oracle.unpack_rows(codes, scales, 16, 32, np.float32).view(np.uint32)
    assert np.array_equal(out.reshape(256, 16), want16)
    assert np.array_equal(out32.reshape(256, 16), want32)


def test_table_index_equals_closed_form(host):
    """The kernels' table-based E2M1 index (one byte-permute lookup) equals the
    closed form for every bf16 magnitude under every closed-form scale, both
    tie rules (host emulation of the byte permute)."""
    assert host.host_check_idx_table() == 0


@pytest.mark.parametrize("sf", [1.0, 6.0, 7.3])
def test_amct_binary32_log2_half_integers(host, oracle, sf):
    """AMCT raw scales whose binary32 log2 may be exactly a half-integer (the
    mantissas near sqrt(2) in every exponent the rule reaches): the kernels'
    window test equals the oracle's log2 rounding.  fp32 blocks hold the max
    and values spread below it."""
    es = np.arange(-30, 127, dtype=np.int64)
    ms = np.arange(0x3504F3 - 64, 0x3504F3 + 64, dtype=np.int64)
    r = (((es[:, None] + 127) << 23) | ms[None, :]).astype(np.uint32).ravel().view(np.float32)
    with np.errstate(over="ignore"):
        amax = (r.astype(np.float64) * sf).astype(np.float32)
    amax = amax[np.isfinite(amax) & (amax < np.float32(2.0 ** 126))]
    g = np.random.default_rng(5)
    x = (amax[:, None] * g.uniform(-1, 1, (len(amax), 32))).astype(np.float32)
    x[:, 0] = amax
    compare(host, oracle, x, 32, "amct", sf)


@pytest.mark.parametrize("sf", [7.3, 5.9, 3.3])
def test_amct_every_bf16_max_other_scale_factors(host, oracle, sf):
    """Every positive finite bf16 block max with scale factors that give raw
    scales with full binary32 mantissas."""
    b = np.arange(1, 0x7F80, dtype=np.uint16)
    x = np.zeros((len(b), 32), np.uint16)
    x[:, 0] = b
    x[:, 1] = b - (b >> 3)
    x[:, 2] = (b >> 1) | 0x8000
    compare(host, oracle, x, 32, "amct", sf)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_amct_sign_of_underflowed_quotient(host, oracle, dtype):
    """Negative values at and around 2^(k-150) under scales 2^k (k = 16..125):
    AMCT's output is +0 where the binary32 quotient x / 2^k underflows, -0
    otherwise; FLOOR keeps -0."""
    rows = []
    for k in range(16, 126):
        t = 2.0 ** (k - 150)
        rows.append([6 * 2.0 ** k, -t, -t * (1 + 2 ** -7), -2 * t, -t / 2, t, -3 * t, -0.75 * t]
                    + [0.0] * 24)
    x32 = np.array(rows, dtype=np.float32)
    x = x32 if dtype == "f32" else W.f32_to_bf16_bits(x32)
    for rule in ("floor", "amct"):
        compare(host, oracle, x, 32, rule)
