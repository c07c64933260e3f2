"""The saturation mask as the pages hand it to torch users (the amct PR page,
fake_quant.py mxfp4_saturation_mask: a bool tensor of x's shape, true where
|x| > 6 * 2^k): mxfp4_saturation_mask and mxfp4_mask_to_bool against the
oracle's clip flags, element for element, on ragged shapes, both rules, both
block sizes, ROW and COL blocking, and into outputs that are and are not
16-byte aligned (the kernel's vector and byte-store paths)."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import CANARY, Guarded, dev, host

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


def make_x(shape, dtype, seed):
    g = np.random.default_rng(seed)
    rows = shape[0]
    a = (g.standard_t(2, size=shape) * np.exp2(g.uniform(-6, 6, (rows,) + (1,) * (len(shape) - 1))))
    a = a.astype(np.float32)
    a.reshape(-1)[::89] = 0.0
    a.reshape(-1)[3::101] = -0.0
    return W.f32_to_bf16_bits(a) if dtype == "bf16" else a


SHAPES = [(1, 1), (1, 17), (7, 33), (37, 91), (64, 4096), (33, 130), (130, 64)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("block", [32, 128])
@pytest.mark.parametrize("rule", ["floor", "amct"])
@pytest.mark.parametrize("axis", ["row", "col"])
@pytest.mark.parametrize("shape", SHAPES)
def test_saturation_mask_matches_oracle(oracle, dtype, block, rule, axis, shape):
    x = make_x(shape, dtype, seed=1000 + 7 * shape[0] + shape[1])
    fn = oracle.qdq_rows if axis == "row" else oracle.qdq_cols
    _, clip, _ = fn(x, block=block, rule=rule)
    ax = M.ROW if axis == "row" else M.COL
    got = M.mxfp4_saturation_mask(dev(x), block=block, rule=rule, axis=ax)
    assert got.dtype == torch.bool and tuple(got.shape) == shape
    np.testing.assert_array_equal(got.cpu().numpy(), clip)


def test_saturation_mask_keeps_leading_dims(oracle):
    x = make_x((6, 5, 77), "bf16", seed=5)
    _, clip, _ = oracle.qdq_rows(x.reshape(30, 77))
    got = M.mxfp4_saturation_mask(dev(x))
    assert tuple(got.shape) == (6, 5, 77)
    np.testing.assert_array_equal(got.cpu().numpy().reshape(30, 77), clip)


@pytest.mark.parametrize("offset", [0, 1, 3, 16])
@pytest.mark.parametrize("layout", ["row", "col"])
def test_mask_to_bool_any_alignment(oracle, offset, layout):
    """The expansion writes exactly rows*cols bytes at out, aligned or not:
    the bytes before and after keep their canary."""
    rows, cols = 45, 203
    x = make_x((rows, cols), "f32", seed=77)
    if layout == "row":
        _, clip, _ = oracle.qdq_rows(x)
        mask = torch.empty(M.row_mask_shape(rows, cols), dtype=torch.int32, device="cuda")
        M.mxfp4_qdq_fwd(dev(x), M.ROW, mask_row=mask)
        ly = M.ROW
    else:
        _, clip, _ = oracle.qdq_cols(x)
        mask = torch.empty(M.col_mask_shape(rows, cols), dtype=torch.int32, device="cuda")
        M.mxfp4_qdq_fwd(dev(x), M.COL, mask_col=mask)
        ly = M.COL
    n = rows * cols
    buf = Guarded((offset + n,), torch.uint8)
    out = buf.t[offset:].view(torch.bool)
    M.mxfp4_mask_to_bool(mask, rows, cols, ly, out=out)
    raw = host(buf.t)
    assert (raw[:offset] == CANARY).all()
    buf.check_tail()
    np.testing.assert_array_equal(raw[offset:], clip.reshape(-1).astype(np.uint8))


def test_mask_to_bool_refuses_short_buffers():
    mask = torch.zeros((4, 2), dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        M.mxfp4_mask_to_bool(mask, 4, 65)                 # needs 3 words per row
    with pytest.raises(ValueError):
        M.mxfp4_mask_to_bool(mask, 4, 64, out=torch.empty(10, dtype=torch.bool, device="cuda"))
    with pytest.raises(ValueError):
        M.mxfp4_mask_to_bool(mask, 4, 64, out=torch.empty(256, dtype=torch.uint8, device="cuda"))
