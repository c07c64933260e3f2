"""Pins for the CPU oracle: checks against what the pages and the mathematics
fix, independent of the oracle's own formulation.

Sources (pages): the amct PR "feat: add MXFP4 QAT fake-quant Linear (with
STE)" -- README section "1. MXFP4 and STE" (scale rule, codebook, clipped STE)
and fake_quant.py (_block_view zero padding, _block_scale, _round_to_e2m1,
_quant_dequant_torch, mxfp4_saturation_mask, _MXFP4FakeQuantSTE); the
hyper-parallel page fake_w4a8_gmm_func.py (group_list counts / cumsum); the
sglang page mxfp4_npu.py (two FP4 codes per byte).

The pins use other formulations than the oracle: nearest-code search by
distance (not midpoint counting), scale exponents by search over k (not
frexp / log2), hand-worked values (tests/golden), direction / grouping
identities, round trips and special cases.
"""
import json
import math
import os

import numpy as np
import pytest

import workloads as W

CODES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def f32(a):
    return np.asarray(a, dtype=np.float32)


def bits32(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


def nearest_code(mag, rule):
    """Brute-force E2M1 snap of |x/scale|: argmin of the distance to the eight
    codes; on an exact tie, the lower code (floor) or the higher one (amct)."""
    mag = np.asarray(mag, dtype=np.float64)
    d = np.abs(mag[..., None] - CODES[None, :])
    best = d.min(axis=-1, keepdims=True)
    hit = d == best
    if rule == "floor":
        idx = np.argmax(hit, axis=-1)                          # first (lowest) minimiser
    else:
        idx = 7 - np.argmax(hit[..., ::-1], axis=-1)           # last (highest) minimiser
    return idx


def expected_from_k(x64, k, rule):
    """Expected QDQ values given the block exponent k, by brute force.  The
    output is negative when the quotient x / 2^k is: exact for floor; for amct
    the binary32 quotient (numpy float32 division), which is +0 or -0 only
    when it underflows."""
    scale = np.ldexp(1.0, k)
    idx = nearest_code(np.abs(x64) / scale, rule)
    q = CODES[idx] * scale
    if rule == "floor":
        quot = x64 / scale
    else:
        with np.errstate(under="ignore"):
            quot = (np.asarray(x64, np.float32) / np.asarray(scale, np.float32)).astype(np.float64)
    q = np.where(quot < 0, -q, q)                              # -0.0 for a negative quotient
    q = np.where(quot == 0, 0.0, q)                            # sign(+-0) = 0 -> +0
    return q, idx


def search_k_floor(amax):
    """Unique k with 4*2^k <= amax < 8*2^k, clamped at -127 (amax = 0 -> -127)."""
    amax = np.asarray(amax, dtype=np.float64)
    out = np.full(amax.shape, -127, dtype=np.int64)
    for k in range(-160, 130):
        lo, hi = math.ldexp(4.0, k), math.ldexp(8.0, k)
        out = np.where((amax >= lo) & (amax < hi), max(k, -127), out)
    return out


def search_k_nearest(r32):
    """k with 2^(2k-1) <= r^2 < 2^(2k+1) (i.e. |log2 r - k| < 1/2), by search.
    r^2 of a 24-bit r is exact in double."""
    r = np.asarray(r32, dtype=np.float64)
    r2 = r * r
    out = np.full(r.shape, 10 ** 6, dtype=np.int64)
    for k in range(-150, 130):
        lo, hi = math.ldexp(1.0, 2 * k - 1), math.ldexp(1.0, 2 * k + 1)
        out = np.where((r2 >= lo) & (r2 < hi), k, out)
    assert (out != 10 ** 6).all()
    return out


_LN2 = None


def binary32_log2_is_half(r):
    """Whether log2(r), rounded to the nearest binary32, is exactly a
    half-integer e + 1/2, decided with 60-digit decimal logarithms: true iff
    |log2 r - (e + 1/2)| is below half a binary32 ulp of e + 1/2 (log2 r is
    irrational near there, so it never equals the boundary)."""
    global _LN2
    from decimal import Decimal, localcontext
    with localcontext() as ctx:
        ctx.prec = 60
        if _LN2 is None:
            _LN2 = Decimal(2).ln()
        lg = Decimal(float(r)).ln() / _LN2
        t = Decimal(math.floor(math.log2(float(r)))) + Decimal("0.5")
        j = math.floor(math.log2(abs(float(t))))
        return abs(lg - t) < Decimal(2) ** (j - 24), int(t - Decimal("0.5"))


def k_amct_pages(r32):
    """The pages' AMCT exponent round(fl32(log2 r)) (torch.round: halves to
    even): the nearest integer to log2 r by search, except where the binary32
    log2 is exactly a half-integer e + 1/2, which goes to the even one of e,
    e + 1.  Candidates are found with double log2 (within 2^-14 of a half) and
    decided exactly by binary32_log2_is_half."""
    r = np.asarray(r32, dtype=np.float32)
    out = search_k_nearest(r)
    lg = np.log2(r.astype(np.float64))
    near = np.abs(lg - np.floor(lg) - 0.5) < 2.0 ** -14
    for i in np.flatnonzero(near.ravel()):
        half, e = binary32_log2_is_half(r.ravel()[i])
        if half:
            out.ravel()[i] = e + (e & 1)
    return out


def all_positive_finite_bf16():
    b = np.arange(1, 0x7F80, dtype=np.uint16)
    return b, W.bf16_bits_to_f32(b)


# ---------------------------------------------------------------- snap pins

@pytest.mark.parametrize("rule", ["floor", "amct"])
@pytest.mark.parametrize("k", [-20, -6, 0, 5, 100])
def test_snap_bruteforce_all_bf16_magnitudes(oracle, rule, k):
    """Every bf16 value |v| <= 6*2^k in a block whose max is 6*2^k (scale 2^k in
    both rules) snaps to the nearest code by distance, with the rule's tie."""
    scale = 2.0 ** k
    b, v = all_positive_finite_bf16()
    v = v[v <= 6 * scale].astype(np.float64)
    vals = np.concatenate([v, -v, [0.0]])
    n = len(vals)
    per = 31
    nrows = -(-n // per)
    blocks = np.zeros((nrows, 32), np.float64)
    blocks[:, 0] = 6 * scale
    flat = np.zeros(nrows * per)
    flat[:n] = vals
    blocks[:, 1:] = flat.reshape(nrows, per)
    xb = W.f32_to_bf16_bits(blocks.astype(np.float32))
    assert (W.bf16_bits_to_f32(xb) == blocks.astype(np.float32)).all()  # exact data
    y, clip, e8 = oracle.qdq_rows(xb, 32, rule)
    assert (e8.astype(int) - 127 == k).all()
    q, _ = expected_from_k(blocks, np.full(blocks.shape, k), rule)
    assert np.array_equal(y, W.f32_to_bf16_bits(q.astype(np.float32)))
    assert not clip.any()


@pytest.mark.parametrize("rule,ks", [("floor", [-127, -30, -6, 0, 20]), ("amct", [-30, -6, 0, 20])])
def test_midpoint_ties(oracle, rule, ks):
    """Exact midpoints m*2^k go to the lower code under floor and to the higher
    one under amct; their float neighbours go to the nearer code in both."""
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    lower = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0]
    upper = [0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for k in ks:
        s = 2.0 ** k
        row = [6 * s] + [m * s for m in mids] + [-m * s for m in mids]
        nb = [float(np.nextafter(np.float32(m * s), np.float32(0))) for m in mids]
        na = [float(np.nextafter(np.float32(m * s), np.float32(np.inf))) for m in mids]
        row += nb + na
        x = f32([row + [0.0] * (32 - len(row))])
        y, _, e8 = oracle.qdq_rows(x, 32, rule)
        assert int(e8[0, 0]) - 127 == k
        got = y[0].astype(np.float64) / s
        want_tie = upper if rule == "amct" else lower
        assert list(got[1:8]) == want_tie
        assert list(got[8:15]) == [-v for v in want_tie]
        assert list(got[15:22]) == lower   # just below: nearer to the lower code
        assert list(got[22:29]) == upper   # just above: nearer to the upper code


@pytest.mark.parametrize("rule", ["floor", "amct"])
@pytest.mark.parametrize("k", [-127 + 97, -3, 0, 11])
def test_codebook_fixed_points(oracle, rule, k):
    """Every signed code c*2^k in a block with max 6*2^k maps to itself."""
    s = 2.0 ** k
    row = [6 * s] + [c * s for c in CODES] + [-c * s for c in CODES[1:]]
    x = f32([row + [0.0] * (32 - len(row))])
    y, clip, _ = oracle.qdq_rows(x, 32, rule)
    assert np.array_equal(bits32(y), bits32(x))
    assert not clip.any()


# --------------------------------------------------------------- scale pins

def test_floor_scale_exhaustive_bf16(oracle):
    """FLOOR exponent: for every positive finite bf16 amax, e8m0-127 equals the
    unique k with 4*2^k <= amax < 8*2^k (clamped at -127)."""
    b, v = all_positive_finite_bf16()
    x = np.zeros((len(b), 32), np.uint16)
    x[:, 5] = b
    _, _, e8 = oracle.qdq_rows(x, 32, "floor")
    assert np.array_equal(e8[:, 0].astype(np.int64) - 127, search_k_floor(v))


@pytest.mark.parametrize("sf", [6.0, 4.0, 7.3])
def test_amct_scale_exhaustive_bf16(oracle, sf):
    """AMCT exponent: round(fl32(log2(max(fl32(amax/sf), 2^-30)))), checked
    through |log2 r - k| < 1/2  <=>  2^(2k-1) <= r^2 < 2^(2k+1) away from the
    binary32 half-integers, which decimal logarithms decide (k_amct_pages)."""
    b, v = all_positive_finite_bf16()
    r = v / np.float32(sf)
    keep = r < np.float32(2.0 ** 126)
    b, v, r = b[keep], v[keep], r[keep]
    r = np.maximum(r, np.float32(2.0 ** -30))
    x = np.zeros((len(b), 32), np.uint16)
    x[:, 31] = b
    _, _, e8 = oracle.qdq_rows(x, 32, "amct", sf)
    assert np.array_equal(e8[:, 0].astype(np.int64) - 127, k_amct_pages(r))


def test_amct_scale_random_fp32(oracle):
    g = np.random.default_rng(11)
    v = np.exp(g.uniform(-60, 60, 200000)).astype(np.float32)
    x = np.zeros((len(v), 32), np.float32)
    x[:, 0] = v
    _, _, e8 = oracle.qdq_rows(x, 32, "amct")
    r = np.maximum(v / np.float32(6.0), np.float32(2.0 ** -30))
    assert np.array_equal(e8[:, 0].astype(np.int64) - 127, k_amct_pages(r))


def _window_r():
    """Every binary32 r = 2^e * m with the mantissa field within 112 of the
    one nearest sqrt(2), for every exponent the AMCT rule reaches."""
    es = np.arange(-30, 128, dtype=np.int64)
    ms = np.arange(0x3504F3 - 56, 0x3504F3 + 56, dtype=np.int64)
    bits = (((es[:, None] + 127) << 23) | ms[None, :]).astype(np.uint32).ravel()
    return bits.view(np.float32)


def test_amct_binary32_log2_half_integers(oracle):
    """Where log2 r rounded to binary32 is exactly e + 1/2 (a window of
    mantissas around sqrt(2) that widens with |e|), the pages' torch.round
    sends it to the even integer; elsewhere k is the nearest integer.  Blocks
    with max r and scale_factor 1 give r itself as the raw scale."""
    r = _window_r()
    x = np.zeros((len(r), 32), np.float32)
    x[:, 3] = r
    _, _, e8 = oracle.qdq_rows(x, 32, "amct", 1.0)
    want = k_amct_pages(r)
    assert np.array_equal(e8[:, 0].astype(np.int64) - 127, want)
    # the windows are not empty: in every exponent at least one r has a binary32
    # log2 that is a half-integer, and about half of those differ from the
    # exact nearest integer (odd e rounds up, even e down)
    differs = want != search_k_nearest(r)
    assert 100 < differs.sum() < len(r) // 2
    e = (r.view(np.uint32) >> 23).astype(np.int64) - 127
    assert set(e[differs] % 2) == {0, 1}


def test_amct_scale_matches_torch_binary32_pipeline(oracle):
    """Cross-check, not a pin: the raw-scale rounding of the pages' code run in
    torch on float32 tensors (clamp(amax / sf, 2^-30), log2, round) agrees
    with the oracle on the window values and on random fp32 maxima."""
    torch = pytest.importorskip("torch")
    g = np.random.default_rng(17)
    wr = _window_r()
    wr = wr[wr < np.float32(2.0 ** 124)]                 # 6 r stays finite
    v = np.concatenate([wr * np.float32(6.0), np.exp(g.uniform(-60, 60, 50000)).astype(np.float32)])
    x = np.zeros((len(v), 32), np.float32)
    x[:, 9] = v
    _, _, e8 = oracle.qdq_rows(x, 32, "amct")
    t = torch.from_numpy(v)
    k = torch.round(torch.log2(torch.clamp(t / 6.0, min=2.0 ** -30))).to(torch.int64).numpy()
    assert np.array_equal(e8[:, 0].astype(np.int64) - 127, k)


def test_floor_scale_random_fp32(oracle):
    g = np.random.default_rng(12)
    v = np.exp(g.uniform(-87, 88, 200000)).astype(np.float32)
    x = np.zeros((len(v), 32), np.float32)
    x[:, 7] = v
    _, _, e8 = oracle.qdq_rows(x, 32, "floor")
    assert np.array_equal(e8[:, 0].astype(np.int64) - 127, search_k_floor(v))


def test_scale_is_power_of_two_bracket(oracle):
    """FLOOR: amax/2^k in [4, 8); AMCT: amax/2^k in [6/sqrt2, 6*sqrt2) (when
    amax/6 >= 2^-30)."""
    g = np.random.default_rng(13)
    x = (g.standard_t(3, size=(4000, 32)) * np.exp(g.uniform(-20, 20, (4000, 1)))).astype(np.float32)
    amax = np.abs(x.astype(np.float64)).max(axis=1)
    _, _, e8 = oracle.qdq_rows(x, 32, "floor")
    ratio = amax / np.ldexp(1.0, e8[:, 0].astype(int) - 127)
    assert ((ratio >= 4) & (ratio < 8)).all()
    _, _, e8a = oracle.qdq_rows(x, 32, "amct")
    ratio = amax / np.ldexp(1.0, e8a[:, 0].astype(int) - 127)
    assert ((ratio >= 6 / math.sqrt(2) * (1 - 1e-7)) & (ratio < 6 * math.sqrt(2) * (1 + 1e-7))).all()


# ----------------------------------------------------- clip, mask, invariants

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_block_max_clipping(oracle, dtype):
    """FLOOR: a block max in (6*2^k, 8*2^k) is clipped to 6*2^k and masked; a max
    of exactly 6*2^k is kept and not masked."""
    rows = []
    for k in (-40, -3, 0, 9):
        s = 2.0 ** k
        for m in (6.0, 6.25, 6.5, 7.0, 7.75, 7.96875):
            rows.append([m * s, -0.5 * s, 1.0 * s] + [0.0] * 29)
    x32 = f32(rows)
    x = x32 if dtype == "f32" else W.f32_to_bf16_bits(x32)
    y, clip, e8 = oracle.qdq_rows(x, 32, "floor")
    yv = y if dtype == "f32" else W.bf16_bits_to_f32(y)
    for i, r in enumerate(rows):
        k = int(e8[i, 0]) - 127
        assert r[0] >= 4 * 2.0 ** k and r[0] < 8 * 2.0 ** k
        assert yv[i, 0] == 6 * 2.0 ** k
        assert clip[i, 0] == (r[0] > 6 * 2.0 ** k)
        assert not clip[i, 1:].any()


@pytest.mark.parametrize("rule", ["floor", "amct"])
@pytest.mark.parametrize("block", [32, 128])
def test_invariants_random_heavy_tailed(oracle, rule, block):
    """On heavy-tailed data with ragged rows: every output is the brute-force
    nearest code times the block scale (or the clip value 6*2^k), the mask is
    exactly |x| > 6*2^k, and the scale matches the rule's search."""
    g = np.random.default_rng(21)
    cols = 3 * block + 17
    x = (g.standard_t(3, size=(64, cols)) * np.exp(g.uniform(-10, 10, (64, 1)))).astype(np.float32)
    x[5, :block] = 0.0
    y, clip, e8 = oracle.qdq_rows(x, block, rule)
    x64 = x.astype(np.float64)
    kfull = np.repeat(e8.astype(np.int64) - 127, block, axis=1)[:, :cols]
    # scale search per block
    pad = (-cols) % block
    xp = np.pad(np.abs(x64), ((0, 0), (0, pad))).reshape(64, -1, block).max(axis=2)
    if rule == "floor":
        assert np.array_equal(e8.astype(np.int64) - 127, search_k_floor(xp))
    else:
        r = np.maximum(xp.astype(np.float32) / np.float32(6.0), np.float32(2.0 ** -30))
        assert np.array_equal(e8.astype(np.int64) - 127, k_amct_pages(r))
    q, idx = expected_from_k(x64, kfull, rule)
    assert np.array_equal(bits32(y), bits32(q.astype(np.float32)))
    assert np.array_equal(clip, np.abs(x64) > 6 * np.ldexp(1.0, kfull))
    assert (np.abs(y) <= 6 * np.ldexp(1.0, kfull)).all()


def test_hand_worked_golden(oracle):
    """Values worked out by hand from the pages' definitions (tests/golden)."""
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        if "x_exact" in case:
            xs = [float.fromhex(v) for v in case["x_exact"]]
        else:
            xs = [float(v) for v in case["x"]]
        n = len(xs)
        x = f32([xs + [0.0] * (32 - n)])
        for rule in ("floor", "amct"):
            want = case[rule]
            y, clip, e8 = oracle.qdq_rows(x, 32, rule)
            wy = [float.fromhex(v) if v.startswith(("0x", "-0x")) else float(v) for v in want["y"]]
            assert list(bits32(y[0, :n])) == list(bits32(f32(wy))), (case["name"], rule)
            assert list(clip[0, :n].astype(int)) == want["mask"], (case["name"], rule)
            assert int(e8[0, 0]) == want["e8m0"], (case["name"], rule)


# ----------------------------------------------------------- special cases

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_zero_blocks(oracle, dtype):
    x32 = np.zeros((3, 64), np.float32)
    x32[1] = -0.0
    x32[2, ::2] = -0.0
    x = x32 if dtype == "f32" else W.f32_to_bf16_bits(x32)
    for rule, byte in (("floor", 0), ("amct", 97)):
        y, clip, e8 = oracle.qdq_rows(x, 32, rule)
        assert (y.view(np.uint32 if dtype == "f32" else np.uint16) == 0).all()
        assert not clip.any()
        assert (e8 == byte).all()


def test_signed_zero_rules(oracle):
    x = f32([[4.0, -1e-3, -0.0, 1e-3, -0.2, 0.0] + [0.0] * 26])
    for rule in ("floor", "amct"):
        y, _, _ = oracle.qdq_rows(x, 32, rule)
        b = bits32(y[0])
        assert b[1] == 0x80000000      # negative value snapping to 0 -> -0.0
        assert b[2] == 0               # -0.0 -> +0.0
        assert b[3] == 0 and b[5] == 0
        if rule == "floor":            # (amct's scale 2^-1 gives -0.2 -> -0.25)
            assert b[4] == 0x80000000


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_amct_sign_of_underflowed_quotient(oracle, dtype):
    """AMCT takes torch.sign of the binary32 quotient x / 2^k: it is zero, and
    the output +0.0, when |x| <= 2^(k-150) (at 2^(k-150) exactly the quotient
    is half the smallest subnormal and rounds to even, i.e. to 0); FLOOR keeps
    the exact sign, -0.0.  Blocks with max 6 * 2^k (scale 2^k in both rules)
    for k from 16 to 125 (6 * 2^125 is near the top of the range) hold
    -2^(k-150) scaled by 1, 1 + 2^-7, 2, 1/2."""
    rows = []
    for k in range(16, 126):
        t = 2.0 ** (k - 150)
        rows.append([6 * 2.0 ** k, -t, -t * (1 + 2 ** -7), -2 * t, -t / 2, t] + [0.0] * 26)
    x32 = np.array(rows, dtype=np.float32)            # values below the dtype's range flush to 0
    x = x32 if dtype == "f32" else W.f32_to_bf16_bits(x32)
    xv = (x if dtype == "f32" else W.bf16_bits_to_f32(x)).astype(np.float64)
    for rule in ("floor", "amct"):
        y, _, e8 = oracle.qdq_rows(x, 32, rule)
        assert (e8[:, 0].astype(int) - 127 == np.arange(16, 126)).all()
        ys = (y.view(np.uint32) >> 31) if dtype == "f32" else (y >> 15)
        neg = xv < 0
        if rule == "floor":
            want = neg
        else:
            lim = np.ldexp(1.0, np.arange(16, 126) - 150)[:, None]
            want = neg & (np.abs(xv) > lim)
        assert np.array_equal(ys.astype(bool), want), rule
        assert (y.view(np.uint32 if dtype == "f32" else np.uint16)[:, 1:] & (0x7FFFFFFF if dtype == "f32" else 0x7FFF) == 0).all()
    # both outcomes occur under amct in every dtype
    assert want.any() and (neg & ~want).any()


def test_subnormal_outputs_bf16(oracle):
    """k = -127: the smallest codes 0.5*2^-127 = 2^-128 are bf16 subnormals."""
    s = 2.0 ** -127
    vals = [6 * s, 0.5 * s, -0.5 * s, 1.5 * s, 0.3 * s]
    x = W.f32_to_bf16_bits(f32([vals + [0.0] * 27]))
    y, clip, e8 = oracle.qdq_rows(x, 32, "floor")
    assert e8[0, 0] == 0
    got = W.bf16_bits_to_f32(y[0, :5]).astype(np.float64) / s
    assert list(got) == [6.0, 0.5, -0.5, 1.5, 0.5]
    assert y[0, 1] == 0x0020       # 2^-128 as a bf16 subnormal


def test_idempotence(oracle):
    """FLOOR QDQ is idempotent (up to -0.0 -> +0.0); AMCT is not (block max 4
    re-scales to 2^-1 and clips to 3)."""
    g = np.random.default_rng(31)
    x = W.f32_to_bf16_bits((g.standard_t(3, size=(256, 96)) * 0.3).astype(np.float32))
    y1, _, _ = oracle.qdq_rows(x, 32, "floor")
    y2, _, _ = oracle.qdq_rows(y1, 32, "floor")
    assert np.array_equal(y2, np.where(y1 == 0x8000, 0, y1).astype(np.uint16))
    xa = f32([[4.0, 1.0] + [0.0] * 30])
    ya, _, _ = oracle.qdq_rows(xa, 32, "amct")
    assert ya[0, 0] == 3.0 and ya[0, 1] == 1.0


# ---------------------------------------------------- directions and groups

@pytest.mark.parametrize("block", [32, 128])
@pytest.mark.parametrize("rule", ["floor", "amct"])
def test_columns_are_rows_of_transpose(oracle, block, rule):
    g = np.random.default_rng(41)
    x = W.f32_to_bf16_bits((g.standard_t(3, size=(block * 2 + 9, 70))).astype(np.float32))
    yc, cc, ec = oracle.qdq_cols(x, block, rule)
    yr, cr, er = oracle.qdq_rows(np.ascontiguousarray(x.T), block, rule)
    assert np.array_equal(yc, yr.T) and np.array_equal(cc, cr.T) and np.array_equal(ec, er.T)


def test_grouped_aligned_equals_columnwise(oracle):
    g = np.random.default_rng(42)
    x = W.f32_to_bf16_bits(g.standard_normal((320, 40)).astype(np.float32))
    counts = np.array([64, 0, 96, 32, 128], np.int64)
    yg, cg, eg = oracle.grouped_cols(x, counts, 32)
    yc, cc, ec = oracle.qdq_cols(x, 32)
    assert np.array_equal(yg, yc) and np.array_equal(cg, cc) and np.array_equal(eg, ec)


@pytest.mark.parametrize("block", [32, 128])
def test_grouped_equals_per_group_slices(oracle, block):
    g = np.random.default_rng(43)
    x = W.f32_to_bf16_bits((g.standard_t(4, size=(700, 24))).astype(np.float32))
    counts = W.ragged_counts(700, 6, seed=3, zero_groups=1)
    yg, cg, eg = oracle.grouped_cols(x, counts, block)
    ends = np.cumsum(counts)
    yg2, cg2, eg2 = oracle.grouped_cols(x, ends, block, list_type=0)
    assert np.array_equal(yg, yg2) and np.array_equal(cg, cg2) and np.array_equal(eg, eg2)
    start, brow = 0, 0
    for c in counts:
        ys, cs, es = oracle.qdq_cols(x[start:start + c], block)
        assert np.array_equal(yg[start:start + c], ys)
        assert np.array_equal(cg[start:start + c], cs)
        nb = es.shape[0]
        assert np.array_equal(eg[brow:brow + nb], es)
        start += c
        brow += nb
    assert brow == eg.shape[0]


def test_grouped_rejects_inconsistent_lists(oracle):
    x = np.zeros((10, 4), np.uint16)
    with pytest.raises(ValueError):
        oracle.grouped_cols(x, [5, 6], 32)
    with pytest.raises(ValueError):
        oracle.grouped_cols(x, [6, 4], 32, list_type=0)


# ------------------------------------------------------------- pack and STE

@pytest.mark.parametrize("block", [32, 128])
@pytest.mark.parametrize("rule", ["floor", "amct"])
def test_pack_roundtrip(oracle, block, rule):
    g = np.random.default_rng(51)
    cols = 2 * block + 11
    x32 = (g.standard_t(3, size=(33, cols)) * 0.02).astype(np.float32)
    x32[3, :5] = [-1e-9, -0.0, 0.0, 1e-9, -6.0]
    x = W.f32_to_bf16_bits(x32)
    codes, sc = oracle.pack_rows(x, block, rule)
    y, _, e8 = oracle.qdq_rows(x, block, rule)
    assert np.array_equal(sc, e8)
    assert np.array_equal(oracle.unpack_rows(codes, sc, cols, block), y)
    assert codes.shape == (33, (cols + 1) // 2)
    assert (codes[:, -1] >> 4 == 0).all()                       # odd row: last high nibble empty
    assert codes[3, 0] & 0x0F == 0x8                            # -tiny -> -0 code (0b1000)
    assert codes[3, 0] >> 4 == 0x0                              # -0.0 -> +0 code


def test_pack_nibble_order_and_codes(oracle):
    """Low nibble = even element; magnitude bits = index into the codebook."""
    s = 1.0
    vals = [6.0, -6.0, 0.5, -0.5, 1.5, 3.0, 0.0, 4.0]
    x = f32([vals + [0.0] * 24])
    codes, sc = oracle.pack_rows(x, 32, "floor")
    assert sc[0, 0] == 127
    assert list(codes[0, :4]) == [0x7 | (0xF << 4), 0x1 | (0x9 << 4), 0x3 | (0x5 << 4), 0x0 | (0x6 << 4)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_unpack_every_nibble_and_scale_byte(oracle, dtype):
    """Decoding is (-1)^s * code * 2^(e8 - 127) for every nibble and every E8M0
    byte: exact (all such values fit fp32 and bf16, subnormals included) up to
    overflow, which gives +-inf (code * 2^(e8-127) > max finite)."""
    nib = np.arange(16, dtype=np.uint8)
    codes = np.repeat((nib | (nib << 4))[None, :], 256, axis=0)        # 256 x 16 bytes
    codes = np.ascontiguousarray(codes[:, :16])
    scales = np.arange(256, dtype=np.uint8)[:, None]                 # one 32-block per row
    want = np.empty((256, 32), np.float64)
    for e8 in range(256):
        for j in range(32):
            n = j // 2
            v = CODES[n & 7] * math.ldexp(1.0, e8 - 127)
            want[e8, j] = -v if n & 8 else v
    with np.errstate(over="ignore"):
        w32 = want.astype(np.float32)
    got = oracle.unpack_rows(codes, scales, 32, 32, np.float32 if dtype == "f32" else np.uint16)
    if dtype == "f32":
        assert np.array_equal(got.view(np.uint32), w32.view(np.uint32))
    else:
        assert np.array_equal(got, W.f32_to_bf16_bits(w32))
        # exactness in bf16: the decoded value round-trips unless it overflowed
        fin = np.isfinite(w32)
        assert np.array_equal(W.bf16_bits_to_f32(got)[fin], w32[fin])
    assert np.isinf(w32[253, 2 * 7]) and np.isfinite(w32[252, 2 * 7])   # 6 * 2^126 overflows


def test_kmajor_hand_worked(oracle):
    """A column [1, -2, 3, 0.5] with 4-row blocks (oracle-only block size):
    amax 3 -> FLOOR k = floor(log2 3) - 2 = -1, scale 0.5, so x/scale =
    [2, -4, 6, 1] -> codes 4, 8|6, 7, 2 -> bytes 0xE4, 0x27, E8M0 126.  The
    second column is all zero: k = -127, E8M0 0, codes 0."""
    x = f32([[1.0, 0.0], [-2.0, 0.0], [3.0, 0.0], [0.5, 0.0]])
    codes, sc, nbt = oracle.pack_kmajor(x, 4, "floor")
    assert nbt == 1
    assert codes.tolist() == [[0xE4, 0x27], [0x00, 0x00]]
    assert sc.tolist() == [[126], [0]]


def _pad_t(a, kp):
    """Transpose and zero-pad the K (row) dimension to kp."""
    t = np.zeros((a.shape[1], kp), a.dtype)
    t[:, :a.shape[0]] = a.T
    return t


@pytest.mark.parametrize("block", [32, 128])
@pytest.mark.parametrize("rule", ["floor", "amct"])
@pytest.mark.parametrize("rows", [64 * 4, 64 * 4 + 37])
def test_kmajor_is_pack_of_padded_transpose(oracle, block, rule, rows):
    """Dense K-major codes are the row-wise packing of x^T with K zero-padded to
    whole blocks (zeros never change a block max and encode as +0), and they
    decode to the column-wise QDQ values."""
    g = np.random.default_rng(45)
    x = W.f32_to_bf16_bits((g.standard_t(3, size=(rows, 20)) * 0.1).astype(np.float32))
    codes, sc, nbt = oracle.pack_kmajor(x, block, rule)
    kp = nbt * block
    assert nbt == -(-rows // block)
    c2, s2 = oracle.pack_rows(_pad_t(x, kp), block, rule)
    assert np.array_equal(codes, c2) and np.array_equal(sc, s2)
    yc, _, ec = oracle.qdq_cols(x, block, rule)
    assert np.array_equal(sc, ec.T)
    dec = oracle.unpack_rows(codes, sc, kp, block)
    assert np.array_equal(dec[:, :rows], yc.T)
    assert (dec[:, rows:] == 0).all()


@pytest.mark.parametrize("block", [32, 128])
def test_kmajor_grouped_is_per_group_pack(oracle, block):
    """Grouped K-major: each group's slab packed on its own (K zero-padded to
    whole blocks), concatenated along K; decodes to grouped_cols' values."""
    g = np.random.default_rng(46)
    x = W.f32_to_bf16_bits((g.standard_t(4, size=(700, 12))).astype(np.float32))
    counts = W.ragged_counts(700, 6, seed=5, zero_groups=1)
    kb = -(-700 // block) + len(counts) - 1
    codes, sc, nbt = oracle.pack_kmajor(x, block, "floor", group_list=counts, k_blocks=kb)
    codes0, sc0, _ = oracle.pack_kmajor(x, block, "floor", group_list=np.cumsum(counts),
                                        list_type=0, k_blocks=kb)
    assert np.array_equal(codes, codes0) and np.array_equal(sc, sc0)
    start, t = 0, 0
    for c in counts:
        nb = -(-int(c) // block)
        if nb:
            c2, s2 = oracle.pack_rows(_pad_t(x[start:start + c], nb * block), block)
            assert np.array_equal(codes[:, t * block // 2:(t + nb) * block // 2], c2)
            assert np.array_equal(sc[:, t:t + nb], s2)
        start += int(c)
        t += nb
    assert t == nbt <= kb
    assert (codes[:, nbt * block // 2:] == 0xA5).all() and (sc[:, nbt:] == 0xA5).all()
    yg, _, eg = oracle.grouped_cols(x, counts, block)
    assert np.array_equal(sc[:, :nbt], eg.T)
    dec = oracle.unpack_rows(np.ascontiguousarray(codes[:, :nbt * block // 2]),
                             np.ascontiguousarray(sc[:, :nbt]), nbt * block, block)
    start, t = 0, 0
    for c in counts:
        c = int(c)
        if c:
            assert np.array_equal(dec[:, t * block:t * block + c], yg[start:start + c].T)
            assert (dec[:, t * block + c:(t + -(-c // block)) * block] == 0).all()
        start += c
        t += -(-c // block)


def test_kmajor_rejects_bad_sizes(oracle):
    x = np.zeros((70, 4), np.uint16)
    with pytest.raises(ValueError):
        oracle.pack_kmajor(x, 32, k_blocks=2)                  # needs 3 block-rows
    with pytest.raises(ValueError):
        oracle.pack_kmajor(x, 32, group_list=[30, 41], k_blocks=4)
    c, s, nbt = oracle.pack_kmajor(x, 32, group_list=[1, 0, 69], k_blocks=4)
    assert nbt == 4


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ste_backward(oracle, dtype):
    g = np.random.default_rng(61)
    x32 = (g.standard_t(3, size=(16, 96)) * 0.02).astype(np.float32)
    x = x32 if dtype == "f32" else W.f32_to_bf16_bits(x32)
    _, clip, _ = oracle.qdq_rows(x, 32, "floor")
    assert clip.any()
    ones32 = np.ones_like(x32)
    ones = ones32 if dtype == "f32" else W.f32_to_bf16_bits(ones32)
    gin = oracle.ste_bwd(ones, clip)
    gv = gin if dtype == "f32" else W.bf16_bits_to_f32(gin)
    assert np.array_equal(gv, 1.0 - clip.astype(np.float32))
    up32 = g.standard_normal(x32.shape).astype(np.float32)
    up32[0, :4] = -0.0
    up = up32 if dtype == "f32" else W.f32_to_bf16_bits(up32)
    assert np.array_equal(oracle.ste_bwd(up), up)                # plain STE: identity
    masked = oracle.ste_bwd(up, clip)
    zero = np.zeros((), up.dtype)
    assert np.array_equal(masked, np.where(clip, zero, up))     # +0 where masked


def test_clip_fraction_statistic(oracle):
    """Soft check of the README remark that the block max is clipped about half
    of the time under the round-to-nearest scale: for log-uniform block maxima
    the clipped fraction is ~0.50 (AMCT) and ~0.415 (FLOOR)."""
    g = np.random.default_rng(71)
    n = 200000
    amax = np.exp2(g.uniform(-8, 8, n)).astype(np.float32)
    x = np.zeros((n, 32), np.float32)
    x[:, 0] = amax
    _, ca, _ = oracle.qdq_rows(x, 32, "amct")
    _, cf, _ = oracle.qdq_rows(x, 32, "floor")
    assert abs(ca[:, 0].mean() - 0.5) < 0.01
    assert abs(cf[:, 0].mean() - math.log2(8 / 6)) < 0.01


# ------------------------------------------------------------- MXFP8 (OCP MX)

def fp8_table(fmt):
    """Value of every non-NaN, finite fp8 code (decoded from the bit fields)."""
    mb, bias = (3, 7) if fmt == "e4m3" else (2, 15)
    vals = {}
    for c in range(256):
        s, ef, m = c >> 7, (c & 0x7F) >> mb, c & ((1 << mb) - 1)
        if fmt == "e4m3" and (c & 0x7F) == 0x7F:
            continue                                   # NaN
        if fmt == "e5m2" and ef == 31:
            continue                                   # inf / NaN
        v = (m / (1 << mb)) * 2.0 ** (1 - bias) if ef == 0 else (1 + m / (1 << mb)) * 2.0 ** (ef - bias)
        vals[c] = -v if s else v
    return vals


def fp8_nearest(v, fmt):
    """Brute-force RNE: nearest code by value, ties to the even code, saturated
    at the largest finite value; zero keeps the sign of v."""
    tab = fp8_table(fmt)
    codes = np.array([c for c in tab if c < 0x80], np.int64)
    mags = np.array([tab[c] for c in codes])
    a = np.minimum(np.abs(v), mags.max())
    d = np.abs(a[:, None] - mags[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    even = cand & ((codes[None, :] & 1) == 0)
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    return (codes[pick] | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("j", [0, -5, 20, -118, 100])
def test_mxfp8_every_bf16_value_against_brute_force(oracle, fmt, j):
    """Every bf16 value v with |v| below a block maximum M = 1.5 * 2^j, in a
    block holding M: the scale is 2^(j - emax) and each code is the nearest
    fp8 value of v / scale (ties to even, saturating)."""
    emax = 8 if fmt == "e4m3" else 15
    M = np.float32(1.5 * 2.0 ** j)
    allb = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    v = W.bf16_bits_to_f32(allb)
    v = v[np.isfinite(v) & (np.abs(v) <= M)]
    n = -(-v.size // 31) * 31
    vv = np.zeros(n, np.float32)
    vv[: v.size] = v
    x = np.concatenate([np.full((n // 31, 1), M, np.float32), vv.reshape(-1, 31)], axis=1)
    xb = W.f32_to_bf16_bits(x)
    q, e8 = oracle.mxfp8_rows(xb, fmt)
    k = max(j - emax, -127)                    # the scale exponent's lower clamp
    assert (e8 == k + 127).all()
    want = fp8_nearest(x[:, 1:].astype(np.float64).reshape(-1) / 2.0 ** k, fmt)
    assert np.array_equal(q[:, 1:].reshape(-1), want)


def test_mxfp8_hand_worked(oracle):
    """amax 1.0: k = 0 - 8, scale 2^-8 (E8M0 119); 1.0 -> 256 = 1.0*2^8 -> 0x78;
    0.3 -> 76.8 -> nearest of {72, 80} = 80 = 1.25*2^6 -> 0x6A (sign 0xEA);
    -0.0 -> 0x80; 1e-5 -> 0.00256 -> one subnormal step 2^-9 -> 0x01.
    A block with maximum 1.99 (scaled 509.4) saturates to 448 -> 0x7E."""
    x = np.zeros((2, 32), np.float32)
    x[0, :6] = [1.0, 0.3, -0.3, 0.0, -0.0, 1e-5]
    x[1, 0] = 1.99
    q, e8 = oracle.mxfp8_rows(x, "e4m3")
    assert list(q[0, :6]) == [0x78, 0x6A, 0xEA, 0x00, 0x80, 0x01]
    assert e8[0, 0] == 119 and e8[1, 0] == 119
    assert q[1, 0] == 0x7E


def test_mxfp8_scale_rule_and_decode(oracle):
    """E8M0 byte = floor(log2 amax) - emax + 127, clamped at 0 (zero and tiny
    blocks); decoding the codes gives values within half a code step, or the
    largest normal times the scale where the element saturated."""
    g = np.random.default_rng(81)
    x = (g.standard_t(3, size=(64, 96)) * np.exp2(g.uniform(-30, 30, (64, 1)))).astype(np.float32)
    x[0] = 0.0
    x[1, :] = 2.0 ** -140                      # fp32 subnormal block maximum
    for fmt, emax in (("e4m3", 8), ("e5m2", 15)):
        q, e8 = oracle.mxfp8_rows(x, fmt)
        amax = np.abs(x.reshape(64, 3, 32)).max(axis=2)
        with np.errstate(divide="ignore"):
            want = np.floor(np.log2(amax)) - emax + 127
        want = np.where(np.isfinite(want), want, 0)
        want = np.where(amax > 0, np.maximum(want, 0), 0)
        assert np.array_equal(e8, want.astype(np.uint8))
        y = oracle.mxfp8_decode(q, e8, fmt, np.float32).astype(np.float64)
        step = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(x), 1e-300))) - (3 if fmt == "e4m3" else 2))
        sub = 2.0 ** (e8.astype(np.float64) - 127 + (-9 if fmt == "e4m3" else -16))
        tol = np.maximum(step, np.repeat(sub, 32, axis=1)) / 2
        maxn = 448.0 if fmt == "e4m3" else 57344.0
        scale = np.repeat(2.0 ** (e8.astype(np.float64) - 127), 32, axis=1)
        tol = np.maximum(tol, np.abs(x) - maxn * scale)     # saturated elements
        assert (np.abs(y - x) <= tol * (1 + 1e-12)).all()
        assert (np.abs(y) <= maxn * scale).all()


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_mxfp8_block128(oracle, fmt):
    """Blocks of 128 (the block-128 mode's activation / grad_output
    quantization): the E8M0 byte follows the block-128 maximum wherever in the
    block it sits, each code is the brute-force nearest fp8 value of x / 2^k
    (ties to even, saturating), ragged rows end in a short block, and decoding
    with one scale per 128 elements gives x / 2^k's code times 2^k."""
    emax = 8 if fmt == "e4m3" else 15
    g = np.random.default_rng(83)
    rows, cols = 48, 3 * 128 + 40
    x = (g.standard_t(3, size=(rows, cols)) * np.exp2(g.uniform(-20, 20, (rows, 1)))).astype(np.float32)
    # put each row's largest element in a different 32-element sub-block of its block
    for r in range(rows):
        x[r, 128 + 32 * (r % 4) + 5] = np.abs(x[r]).max() * 3
    q, e8 = oracle.mxfp8_rows(x, fmt, block=128)
    assert e8.shape == (rows, 4)
    pad = np.zeros((rows, 4 * 128), np.float64)
    pad[:, :cols] = np.abs(x)
    amax = pad.reshape(rows, 4, 128).max(axis=2)
    want_e8 = np.maximum(np.floor(np.log2(amax)) - emax + 127, 0).astype(np.uint8)
    assert np.array_equal(e8, want_e8)
    k = np.repeat(e8.astype(np.int64) - 127, 128, axis=1)[:, :cols]
    want = fp8_nearest(x.astype(np.float64).reshape(-1) / np.exp2(k.reshape(-1)), fmt)
    assert np.array_equal(q.reshape(-1), want)
    y = oracle.mxfp8_decode(q, e8, fmt, np.float64, block=128)
    y32 = oracle.mxfp8_decode(q, np.repeat(e8, 4, axis=1)[:, : -(-cols // 32)], fmt, np.float64)
    assert np.array_equal(y, y32)                      # one scale per 128 = the same scale per 32
    tab = fp8_table(fmt)
    vals = np.array([tab[int(c)] for c in want])
    assert np.array_equal(y.reshape(-1), vals * np.exp2(k.reshape(-1)))


# ---- grouped matrix product ---------------------------------------------------

GOLDEN_GMM = os.path.join(os.path.dirname(__file__), "golden", "grouped_matmul.json")


def test_grouped_matmul_hand_worked(oracle):
    with open(GOLDEN_GMM) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        out = oracle.grouped_matmul(np.array(c["left"], float), np.array(c["right"], float),
                                    c["group_list"], c["group_type"], c["list_type"])
        exp = np.array([[np.nan if v is None else v for v in row] for row in c["out"]]
                       if c["group_type"] == 0 else c["out"], float)
        assert np.array_equal(out, exp, equal_nan=True), c["name"]


def _counts_to_ends(counts):
    return np.cumsum(counts)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_grouped_matmul_rows_against_library(oracle, seed):
    """group_type 0: every group's rows equal a library product of that slice
    with the group's own right operand; list types agree; rows past the total
    keep their old values."""
    g = np.random.default_rng(seed)
    M, K, N, G = 37, 23, 11, 5
    counts = g.multinomial(M - 4, np.ones(G) / G)
    counts[2] = 0
    left = g.standard_normal((M, K))
    right = g.standard_normal((G, K, N))
    out = oracle.grouped_matmul(left, right, counts, oracle.GROUP_M, 1)
    out0 = oracle.grouped_matmul(left, right, _counts_to_ends(counts), oracle.GROUP_M, 0)
    assert np.array_equal(out, out0, equal_nan=True)
    s = 0
    for gi, c in enumerate(counts):
        np.testing.assert_allclose(out[s:s + c], left[s:s + c] @ right[gi], rtol=1e-13, atol=1e-13)
        s += c
    assert np.isnan(out[s:]).all()
    one = oracle.grouped_matmul(left, right[1], None, oracle.GROUP_M)
    np.testing.assert_allclose(one, left @ right[1], rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("seed", [0, 1])
def test_grouped_matmul_reduction_against_library(oracle, seed):
    """group_type 2: out[g] is a library product over group g's slice of the
    reduction dimension; the groups' sum is the product over every covered
    index."""
    g = np.random.default_rng(seed)
    M, K, N, G = 13, 41, 9, 4
    counts = g.multinomial(K - 3, np.ones(G) / G)
    counts[0] = 0
    left = g.standard_normal((M, K))
    right = g.standard_normal((K, N))
    out = oracle.grouped_matmul(left, right, counts, oracle.GROUP_K, 1)
    assert out.shape == (G, M, N)
    s = 0
    for gi, c in enumerate(counts):
        np.testing.assert_allclose(out[gi], left[:, s:s + c] @ right[s:s + c], rtol=1e-13, atol=1e-13)
        s += c
    np.testing.assert_allclose(out.sum(0), left[:, :s] @ right[:s], rtol=1e-12, atol=1e-12)
    out0 = oracle.grouped_matmul(left, right, _counts_to_ends(counts), oracle.GROUP_K, 0)
    assert np.array_equal(out, out0)


def test_grouped_matmul_sum_is_exact_beyond_double(oracle):
    """Sums run in extended precision: 2^60 + 1 - 2^60 = 1 in every layout."""
    left = np.array([[2.0 ** 60, 1.0, -(2.0 ** 60)]])
    right = np.ones((3, 1))
    assert oracle.grouped_matmul(left, right[None], [1], oracle.GROUP_M)[0, 0] == 1.0
    assert oracle.grouped_matmul(left, right, [3], oracle.GROUP_K)[0, 0, 0] == 1.0


def test_grouped_matmul_mx_operands_scale_exactly(oracle):
    """On decoded MX operands (MXFP8 rows times MXFP4 rows), raising one
    row's E8M0 byte by one doubles exactly that output row, and raising one
    weight column's byte doubles exactly that output column."""
    g = np.random.default_rng(5)
    M, K, N = 6, 64, 5
    x = W.f32_to_bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    w = W.f32_to_bf16_bits(g.standard_normal((N, K)).astype(np.float32))
    q, sa = oracle.mxfp8_rows(x)
    codes, sb = oracle.pack_rows(w)
    def prod(sa_, sb_):
        a = oracle.mxfp8_decode(q, sa_, "e4m3", np.float64)
        b = oracle.unpack_rows(codes, sb_, K, 32, np.float64)
        return oracle.grouped_matmul(a, b.T.copy()[None], None, oracle.GROUP_M)
    base = prod(sa, sb)
    sa2 = sa.copy()
    sa2[3] += 1
    r = prod(sa2, sb)
    assert np.array_equal(r[3], 2 * base[3]) and np.array_equal(np.delete(r, 3, 0), np.delete(base, 3, 0))
    sb2 = sb.copy()
    sb2[1] += 1
    r = prod(sa, sb2)
    assert np.array_equal(r[:, 1], 2 * base[:, 1]) and np.array_equal(np.delete(r, 1, 1), np.delete(base, 1, 1))


def test_grouped_matmul_rejects_bad_lists(oracle):
    left, right = np.ones((4, 3)), np.ones((2, 3, 2))
    for gl, lt in (([3, 2], 1), ([-1, 5], 1), ([3, 2], 0), ([2, 5], 0)):
        with pytest.raises(ValueError):
            oracle.grouped_matmul(left, right, gl, oracle.GROUP_M, lt)
    with pytest.raises(ValueError):
        oracle.grouped_matmul(left, np.ones((3, 2)), [1, 3], oracle.GROUP_K, 1)


def test_decoders_float64_match_float32(oracle):
    g = np.random.default_rng(8)
    x = W.f32_to_bf16_bits(g.standard_normal((7, 96)).astype(np.float32))
    q, s = oracle.mxfp8_rows(x)
    assert np.array_equal(oracle.mxfp8_decode(q, s, "e4m3", np.float64),
                          oracle.mxfp8_decode(q, s, "e4m3", np.float32).astype(np.float64))
    c, s4 = oracle.pack_rows(x)
    assert np.array_equal(oracle.unpack_rows(c, s4, 96, 32, np.float64),
                          oracle.unpack_rows(c, s4, 96, 32, np.float32).astype(np.float64))


# ---- K-major MXFP8 (grouped column-wise operand of the TN product) ------------------

def test_mxfp8_kmajor_hand_worked(oracle):
    """Three tokens x two columns, groups [2, 1] (E4M3).  Column 0: block {1, 0.5}:
    amax 1 -> k = 0 - 8, e8 119, codes 256 = 2^8 -> 0x78, 128 -> 0x70; block {7}:
    k = 2 - 8, e8 121, 7 * 2^6 = 448 -> 0x7E.  Column 1: block {-3, 100}: k = 6 - 8,
    e8 125, -12 = -1.5 * 2^3 -> 0xD4, 400 lies midway between 384 and 416 -> even
    mantissa -> 384 -> 0x7C; block {0}: e8 0, code 0.  Every other K position of a
    block is padding 0."""
    x = np.array([[1.0, -3.0], [0.5, 100.0], [7.0, 0.0]], np.float32)
    q, s, nbt = oracle.mxfp8_kmajor(x, "e4m3", [2, 1], 1, k_blocks=3)
    assert nbt == 2
    exp_q = np.zeros((2, 64), np.uint8)
    exp_q[0, [0, 1, 32]] = [0x78, 0x70, 0x7E]
    exp_q[1, [0, 1, 32]] = [0xD4, 0x7C, 0x00]
    assert np.array_equal(q[:, :64], exp_q)
    assert (q[:, 64:] == 0xA5).all() and (s[:, 2] == 0xA5).all()   # block-row 2: untouched
    assert np.array_equal(s[:, :2], np.array([[119, 121], [125, 0]], np.uint8))


@pytest.mark.parametrize("rows", [1, 31, 32, 77, 200])
@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_mxfp8_kmajor_is_rows_of_transpose(oracle, rows, fmt):
    """Dense column-wise blocks: the K-major codes are the row-wise MXFP8 of x^T,
    followed by zero padding up to the block-row boundary; the scales agree."""
    g = np.random.default_rng(rows)
    x = W.f32_to_bf16_bits((g.standard_t(3, (rows, 9)) * np.exp2(g.uniform(-20, 20, (1, 9)))).astype(np.float32))
    nb = -(-rows // 32)
    q, s, nbt = oracle.mxfp8_kmajor(x, fmt, k_blocks=nb + 3)
    assert nbt == nb
    qr, sr = oracle.mxfp8_rows(np.ascontiguousarray(W.bf16_bits_to_f32(x).T.astype(np.float32)), fmt)
    assert np.array_equal(q[:, :rows], qr)
    assert (q[:, rows:32 * nb] == 0).all()
    assert np.array_equal(s[:, :nb], sr)
    assert (q[:, 32 * nb:] == 0xA5).all() and (s[:, nb:] == 0xA5).all()


def test_mxfp8_kmajor_grouped_is_per_group(oracle):
    """Grouped blocks restart at every group start: each group's block-rows are
    the dense K-major MXFP8 of that group's rows, placed after the previous
    groups' block-rows; list types agree."""
    g = np.random.default_rng(3)
    counts = np.array([45, 0, 1, 64, 30], np.int64)
    x = W.f32_to_bf16_bits(g.standard_normal((int(counts.sum()) + 5, 11)).astype(np.float32))
    nbt = int(sum(-(-int(c) // 32) for c in counts))
    q, s, n = oracle.mxfp8_kmajor(x, "e4m3", counts, 1, k_blocks=nbt + 2)
    q0, s0, _ = oracle.mxfp8_kmajor(x, "e4m3", np.cumsum(counts), 0, k_blocks=nbt + 2)
    assert n == nbt and np.array_equal(q, q0) and np.array_equal(s, s0)
    r0, b0 = 0, 0
    for c in counts:
        nb = -(-int(c) // 32)
        if c:
            qg, sg, _ = oracle.mxfp8_kmajor(np.ascontiguousarray(x[r0:r0 + c]), "e4m3")
            assert np.array_equal(q[:, 32 * b0:32 * (b0 + nb)], qg)
            assert np.array_equal(s[:, b0:b0 + nb], sg)
        r0 += int(c)
        b0 += nb


def test_mxfp8_kmajor_rejects_bad_sizes(oracle):
    x = np.ones((40, 3), np.float32)
    with pytest.raises(ValueError):
        oracle.mxfp8_kmajor(x, "e4m3", k_blocks=1)               # needs 2 block-rows
    with pytest.raises(ValueError):
        oracle.mxfp8_kmajor(x, "e4m3", [30, 20], 1, k_blocks=4)  # past rows
