"""Seeded synthetic inputs shared by the tests, bench.py and smoke().

This module holds no MXFP4 arithmetic: it only draws numbers (numpy PCG64) and
plants fixed values at known positions.  bf16 tensors are returned as uint16
bit patterns (round-to-nearest-even from float32), fp32 as float32.

The five workloads mirror the shapes of the pages' layers:
  tiny_qat    fp32 weight 32x64 and input 4x64 ~ N(0,1), seed 0 (the PR's
              minimal validation uses Linear(64, 32) and randn(4, 64));
  weight_4k   bf16 4096x4096 ~ N(0, 0.02^2) with 0.1 % outliers +-U(10,50)*0.02,
              1 % all-zero 32-blocks and planted codebook/midpoint blocks;
              upstream gradient bf16 ~ N(0,1);
  act_dual    bf16 16384x8192 Student-t(nu=3) * 0.5;
  moe_grouped bf16 32768x7168 ~ N(0,1), 8 groups, counts ~ multinomial(uniform);
  weight_pack bf16 28672x8192 ~ N(0, 0.02^2) with 0.05 % outliers +-U(5,20)*0.02.
"""
from __future__ import annotations

import numpy as np

SIGMA_W = 0.02

# Values planted into the weight_4k workload (data only): the E2M1 codebook and
# the midpoints between its neighbours, as listed on the pages.
_PLANT_CODES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)
_PLANT_MIDS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def normal_bf16(shape, sigma: float, seed: int) -> np.ndarray:
    g = _rng(seed)
    return f32_to_bf16_bits(g.standard_normal(shape, dtype=np.float32) * np.float32(sigma))


def normal_f32(shape, sigma: float, seed: int) -> np.ndarray:
    g = _rng(seed)
    return (g.standard_normal(shape, dtype=np.float32) * np.float32(sigma)).astype(np.float32)


def student_t_bf16(shape, nu: float, scale: float, seed: int) -> np.ndarray:
    g = _rng(seed)
    return f32_to_bf16_bits((g.standard_t(nu, size=shape) * scale).astype(np.float32))


def _outliers_f32(x: np.ndarray, frac: float, lo: float, hi: float, sigma: float,
                  g: np.random.Generator) -> np.ndarray:
    """Replace a fraction of entries by s*u*sigma, s = +-1, u ~ U(lo, hi)."""
    n = x.size
    k = int(round(n * frac))
    if k == 0:
        return np.zeros(0, np.int64)
    pos = g.choice(n, size=k, replace=False)
    s = np.where(g.random(k) < 0.5, -1.0, 1.0)
    u = g.uniform(lo, hi, size=k)
    x.reshape(-1)[pos] = (s * u * sigma).astype(np.float32)
    return pos


def edge_blocks_f32(block: int = 32):
    """Rows of `block` values exercising ties, codebook points, clipping,
    tiny/subnormal scales and signed zeros.  Returned as a float32 array of
    shape [n_blocks, block] (each row is one block); data only."""
    rows = []
    for j in (-8, -6, -4, 0, 3):
        s = 2.0 ** j
        base = [6.0 * s]
        base += [m * s for m in _PLANT_MIDS] + [-m * s for m in _PLANT_MIDS]
        base += [c * s for c in _PLANT_CODES] + [-c * s for c in _PLANT_CODES]
        rows.append(base)
        # neighbours of every midpoint (one float32 ulp each side)
        nb = [6.0 * s]
        for m in _PLANT_MIDS:
            v = np.float32(m * s)
            nb += [float(np.nextafter(v, np.float32(0))), float(np.nextafter(v, np.float32(np.inf)))]
        rows.append(nb)
        rows.append([7.0 * s] + [((i % 13) - 6) * 0.5 * s for i in range(block - 1)])  # clipped max
        rows.append([4.0 * s, 3.5 * s, -3.0 * s, 2.5 * s, 0.75 * s, -0.25 * s])        # max 4*2^j
        rows.append([-1e-3 * s, -0.0, 0.0, 5.0 * s])                                    # signed zeros
    # tiny / subnormal magnitudes (k at or near the bottom of the E8M0 range)
    for e in (-133, -130, -128, -127, -126, -125, -124, -123, -122, -121, -120, -100):
        s = 2.0 ** e
        rows.append([s * v for v in (7.5, 6.0, 5.0, 3.5, 3.0, 2.5, 1.75, 1.5, 1.25, 1.0,
                                     0.75, 0.5, 0.25, -0.25, -0.75, -1.25, -7.0, 0.0)])
        rows.append([s * (1.0 + i / 16.0) * (-1) ** i for i in range(block)])
    rows.append([0.0] * block)
    rows.append([-0.0] * block)
    out = np.zeros((len(rows), block), np.float32)
    for i, r in enumerate(rows):
        r = r[:block]
        out[i, :len(r)] = np.asarray(r, np.float64).astype(np.float32)
    return out


# ---------------------------------------------------------------- workloads

def tiny_qat(seed: int = 0):
    """fp32 weight 32x64 and fp32 input 4x64 ~ N(0, 1)."""
    g = _rng(seed)
    w = g.standard_normal((32, 64), dtype=np.float32)
    x = g.standard_normal((4, 64), dtype=np.float32)
    return w, x


def weight_4k(seed: int = 2, rows: int = 4096, cols: int = 4096, plant: bool = True,
              with_grad: bool = True):
    """bf16 weight ~ N(0, 0.02^2), 0.1 % outliers +-U(10,50)*0.02, 1 % zero
    32-blocks, planted edge blocks.  Returns (x_bits, grad_bits_or_None, manifest)
    where manifest lists the (row, first_col) of each planted block."""
    g = _rng(seed)
    x = g.standard_normal((rows, cols), dtype=np.float32) * np.float32(SIGMA_W)
    _outliers_f32(x, 1e-3, 10.0, 50.0, SIGMA_W, g)
    nblk = rows * (cols // 32)
    kz = int(round(nblk * 0.01))
    zb = g.choice(nblk, size=kz, replace=False)
    xb = x.reshape(rows, cols // 32, 32)
    xb.reshape(-1, 32)[zb] = 0.0
    manifest = []
    if plant:
        edges = edge_blocks_f32(32)
        # plant one edge block per 64 rows, spread over the columns
        for i, blk in enumerate(edges):
            r = (i * 67) % rows
            c0 = ((i * 29) % (cols // 32)) * 32
            x[r, c0:c0 + 32] = blk
            manifest.append((r, c0))
    grad = None
    if with_grad:
        grad = f32_to_bf16_bits(g.standard_normal((rows, cols), dtype=np.float32))
    return f32_to_bf16_bits(x), grad, manifest


def act_dual(seed: int = 3, rows: int = 16384, cols: int = 8192):
    """bf16 activation, Student-t (nu = 3) scaled by 0.5."""
    return student_t_bf16((rows, cols), 3.0, 0.5, seed)


def moe_grouped(seed: int = 4, rows: int = 32768, cols: int = 7168, groups: int = 8):
    """bf16 N(0,1) activation and int64 per-group row counts (multinomial)."""
    g = _rng(seed)
    counts = g.multinomial(rows, [1.0 / groups] * groups).astype(np.int64)
    x = f32_to_bf16_bits(g.standard_normal((rows, cols), dtype=np.float32))
    return x, counts


def weight_pack(seed: int = 5, rows: int = 28672, cols: int = 8192):
    """bf16 weight ~ N(0, 0.02^2) with 0.05 % outliers +-U(5,20)*0.02."""
    g = _rng(seed)
    x = g.standard_normal((rows, cols), dtype=np.float32) * np.float32(SIGMA_W)
    _outliers_f32(x, 5e-4, 5.0, 20.0, SIGMA_W, g)
    return f32_to_bf16_bits(x)


def moe_expert_weights(seed: int = 6, groups: int = 8, k: int = 7168, n: int = 2048):
    """bf16 expert weights W[g] of shape [k, n] (x @ W[g]), ~ N(0, 0.02^2): the
    weight side of the grouped MoE layer (hidden 7168 -> expert width 2048)."""
    g = _rng(seed)
    w = g.standard_normal((groups, k, n), dtype=np.float32) * np.float32(SIGMA_W)
    return f32_to_bf16_bits(w)


def ragged_counts(rows: int, groups: int, seed: int, zero_groups: int = 0) -> np.ndarray:
    """Random per-group row counts summing to `rows`, some groups empty."""
    g = _rng(seed)
    counts = g.multinomial(rows, [1.0 / groups] * groups).astype(np.int64)
    for z in g.choice(groups, size=min(zero_groups, groups - 1), replace=False):
        counts[(z + 1) % groups] += counts[z]
        counts[z] = 0
    return counts
