"""Batched row-wise calls (mxfp4_qdq_fwd_rows_batch, mxfp4_ste_bwd_rows_batch):
every output of every item equals the single-tensor call's bit for bit and
the oracle's, across dtypes, blocks, rules, the three row layouts (cols a
multiple of the block, of 8, neither), an empty item, and one to eight items
per launch; no byte past an output is written (canaries)."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import Guarded, dev, host, like_bf16_or_f32, unpack_row_bitmap

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


def make(shape, dtype, seed):
    g = np.random.default_rng(seed)
    a = (g.standard_t(3, size=shape) * np.exp2(g.uniform(-6, 6, (shape[0], 1)))).astype(np.float32)
    a.reshape(-1)[::53] = 0.0
    a.reshape(-1)[7::61] = -0.0
    return W.f32_to_bf16_bits(a) if dtype == "bf16" else a


SHAPE_SETS = [
    [(32, 64), (4, 64)],                                     # the tiny QAT layer
    [(5, 256)],
    [(3, 96), (7, 40), (2, 13), (0, 64), (9, 128)],          # flat, rows-vec, rows-scalar, empty
    [(1, 32), (2, 64), (3, 96), (4, 128), (5, 160), (6, 192), (7, 224), (8, 1000)],   # eight items
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("block", [32, 128])
@pytest.mark.parametrize("rule", ["floor", "amct"])
@pytest.mark.parametrize("si", range(len(SHAPE_SETS)))
def test_forward_batch_equals_single_calls_and_oracle(oracle, dtype, block, rule, si):
    shapes = SHAPE_SETS[si]
    xs_np = [make(s, dtype, 100 * si + i) for i, s in enumerate(shapes)]
    xs = [dev(a) for a in xs_np]
    et = like_bf16_or_f32(xs_np[0])
    ys = [Guarded(s, et) for s in shapes]
    ms = [Guarded((s[0], -(-s[1] // 32)), torch.int32) for s in shapes]
    ss = [Guarded((s[0], -(-s[1] // block)), torch.uint8) for s in shapes]
    M.mxfp4_qdq_fwd_rows_batch(xs, [y.t for y in ys], [m.t for m in ms], [c.t for c in ss], block=block, rule=rule)
    torch.cuda.synchronize()
    for i, (s, a) in enumerate(zip(shapes, xs_np)):
        for buf in (ys[i], ms[i], ss[i]):
            buf.check_tail()
        if s[0] * s[1] == 0:
            continue
        y1 = torch.empty(s, dtype=et, device="cuda")
        m1 = torch.empty((s[0], -(-s[1] // 32)), dtype=torch.int32, device="cuda")
        s1 = torch.empty((s[0], -(-s[1] // block)), dtype=torch.uint8, device="cuda")
        M.mxfp4_qdq_fwd(xs[i], M.ROW, y_row=y1, mask_row=m1, scales_row=s1, block=block, rule=rule)
        assert np.array_equal(host(ys[i].t), host(y1))
        assert np.array_equal(host(ms[i].t), host(m1))
        assert np.array_equal(host(ss[i].t), host(s1))
        yo, clip, e8 = oracle.qdq_rows(a, block, rule)
        assert np.array_equal(host(ys[i].t), yo)
        bits, pad_zero = unpack_row_bitmap(host(ms[i].t), s[1])
        assert np.array_equal(bits, clip) and pad_zero
        assert np.array_equal(host(ss[i].t), e8)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("si", range(len(SHAPE_SETS)))
def test_ste_batch_equals_single_calls_and_oracle(oracle, dtype, si):
    shapes = SHAPE_SETS[si]
    xs_np = [make(s, dtype, 7 + i) for i, s in enumerate(shapes)]
    gs_np = [make(s, dtype, 70 + i) for i, s in enumerate(shapes)]
    masks, clips = [], []
    for a, s in zip(xs_np, shapes):
        m = torch.empty((s[0], -(-s[1] // 32)), dtype=torch.int32, device="cuda")
        if s[0] * s[1]:
            M.mxfp4_qdq_fwd(dev(a), M.ROW, mask_row=m)
        masks.append(m)
        clips.append(oracle.qdq_rows(a, 32)[1] if s[0] * s[1] else None)
    # every other item uses the plain STE (no bitmap)
    use = [m if i % 2 == 0 else None for i, m in enumerate(masks)]
    gs = [dev(g) for g in gs_np]
    et = like_bf16_or_f32(gs_np[0])
    gis = [Guarded(s, et) for s in shapes]
    M.mxfp4_ste_bwd_rows_batch(gs, use, [g.t for g in gis])
    torch.cuda.synchronize()
    for i, s in enumerate(shapes):
        gis[i].check_tail()
        if s[0] * s[1] == 0:
            continue
        g1 = torch.empty(s, dtype=et, device="cuda")
        M.mxfp4_ste_bwd(gs[i], use[i], g1)
        assert np.array_equal(host(gis[i].t), host(g1))
        want = oracle.ste_bwd(gs_np[i], clips[i] if use[i] is not None else None)
        assert np.array_equal(host(gis[i].t), want)


def test_ste_batch_in_place():
    x = dev(make((16, 64), "f32", 3))
    m = torch.empty((16, 2), dtype=torch.int32, device="cuda")
    M.mxfp4_qdq_fwd(x, M.ROW, mask_row=m)
    g = dev(make((16, 64), "f32", 4))
    want = g.clone()
    M.mxfp4_ste_bwd(want, m, want)
    g2 = g.clone()
    M.mxfp4_ste_bwd_rows_batch([g, g2], [m, None], [g, g2])     # clipped in place, plain in place
    assert torch.equal(g, want)
    assert torch.equal(g2, dev(make((16, 64), "f32", 4)))


def test_batch_refusals():
    x = torch.zeros((4, 64), device="cuda")
    y = torch.empty_like(x)
    with pytest.raises(ValueError):
        M.mxfp4_qdq_fwd_rows_batch([x] * 9, [torch.empty_like(x) for _ in range(9)])
    with pytest.raises(ValueError):
        M.mxfp4_qdq_fwd_rows_batch([x, x.to(torch.bfloat16)], [y, torch.empty_like(x, dtype=torch.bfloat16)])
    with pytest.raises(ValueError):
        M.mxfp4_qdq_fwd_rows_batch([x, x], [y, y])                 # two items write the same y
    with pytest.raises(ValueError):
        M.mxfp4_qdq_fwd_rows_batch([x], [None])                    # no output
    with pytest.raises(ValueError):
        M.mxfp4_ste_bwd_rows_batch([x, x], [None, None], [y, y])  # shared grad_in
