"""Host-side checks of the Python binding's argument validation (no GPU
needed: every check here runs before the library is loaded or a pointer is
taken).  The C ABI receives bare pointers, so the binding is where an output
buffer smaller than what the kernels write is refused."""
import pytest
import torch

import mxfp4_fake_quantization_amd as M


def t(*shape, dtype=torch.int32):
    return torch.empty(shape, dtype=dtype)


def test_qdq_fwd_refuses_small_outputs():
    x = t(100, 70, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="mask_row"):
        M.mxfp4_qdq_fwd(x, M.ROW, mask_row=t(100, 2))
    with pytest.raises(ValueError, match="scales_row"):
        M.mxfp4_qdq_fwd(x, M.ROW, scales_row=t(100, 2, dtype=torch.uint8))
    with pytest.raises(ValueError, match="mask_col"):
        M.mxfp4_qdq_fwd(x, M.COL, mask_col=t(3, 70))
    with pytest.raises(ValueError, match="scales_col"):
        M.mxfp4_qdq_fwd(x, M.COL, scales_col=t(3, 70, dtype=torch.uint8))
    with pytest.raises(ValueError, match="scales_row"):
        M.mxfp4_qdq_fwd(x, M.ROW, scales_row=t(99, 1, dtype=torch.uint8), block=128)
    with pytest.raises(ValueError):
        M.mxfp4_qdq_fwd(x, M.ROW, y_row=t(100, 69, dtype=torch.bfloat16))


def test_grouped_refuses_small_outputs():
    x = t(300, 64, dtype=torch.bfloat16)
    y = torch.empty_like(x)
    # host list [100, 0, 200]: 4 + 7 = 11 block-rows of 32
    with pytest.raises(ValueError, match="scales"):
        M.mxfp4_grouped_qdq(x, [100, 0, 200], y, scales=t(10, 64, dtype=torch.uint8))
    with pytest.raises(ValueError, match="mask"):
        # a uint8 buffer viewed as int32 holds a quarter of the words needed
        M.mxfp4_grouped_qdq(x, [100, 0, 200], y, mask=t(11, 64, dtype=torch.uint8).view(torch.int32))
    with pytest.raises(ValueError, match="mask"):
        M.mxfp4_ste_bwd(x, t(10, 64), y, layout=M.GROUPED, group_list=[100, 0, 200])
    with pytest.raises(ValueError, match="group_list"):
        M.mxfp4_grouped_qdq(x, None, y)


def test_pack_refuses_small_outputs():
    x = t(9, 77, dtype=torch.float32)
    with pytest.raises(ValueError, match="codes"):
        M.mxfp4_quant_pack(x, t(9, 38, dtype=torch.uint8), t(9, 3, dtype=torch.uint8))
    with pytest.raises(ValueError, match="scales"):
        M.mxfp4_quant_pack(x, t(9, 39, dtype=torch.uint8), t(9, 2, dtype=torch.uint8))
    with pytest.raises(ValueError, match="mask"):
        M.mxfp4_quant_pack(x, t(9, 39, dtype=torch.uint8), t(9, 3, dtype=torch.uint8), mask=t(9, 2))


def test_ste_refuses_small_masks():
    g = t(40, 100, dtype=torch.bfloat16)
    gi = torch.empty_like(g)
    with pytest.raises(ValueError, match="mask"):
        M.mxfp4_ste_bwd(g, t(40, 3), gi, layout=M.ROW)
    with pytest.raises(ValueError, match="mask"):
        M.mxfp4_ste_bwd(g, t(1, 100), gi, layout=M.COL)


def test_grouped_matmul_refuses_missing_groups_and_rows():
    u8 = torch.uint8
    a, asc = t(64, 128, dtype=u8), t(64, 4, dtype=u8)
    b, bsc = t(2, 48, 64, dtype=u8), t(2, 48, 4, dtype=u8)     # 2 experts, N=48, K=128 (fp4)
    c = t(64, 48, dtype=torch.float32)
    with pytest.raises(ValueError, match="one matrix per group"):
        M.mxfp4_grouped_matmul(a, asc, b, bsc, c, group_list=[10, 20, 34])
    with pytest.raises(ValueError, match="a_scales"):
        M.mxfp4_grouped_matmul(a, t(63, 4, dtype=u8), b, bsc, c, group_list=[30, 34])
    with pytest.raises(ValueError, match="b_scales"):
        M.mxfp4_grouped_matmul(a, asc, b, t(2, 47, 4, dtype=u8), c, group_list=[30, 34])
