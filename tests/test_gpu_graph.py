"""The batched row-wise calls captured in a HIP graph (torch.cuda.CUDAGraph
over the C-ABI launches, which enqueue on torch's current stream and
allocate nothing) and replayed: every replay, with new inputs copied into
the captured buffers and eager work in between, equals the eager calls bit
for bit (and the oracle)."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import dev, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_batched_step_graph_replays_match_eager(oracle, dtype):
    import mxfp4_fake_quantization_amd as M
    shapes = [(32, 64), (4, 64), (6, 40)]
    g = np.random.default_rng(11)

    def sample(seed):
        r = np.random.default_rng(seed)
        out = []
        for s in shapes:
            a = (r.standard_t(3, size=s) * 0.5).astype(np.float32)
            out.append(W.f32_to_bf16_bits(a) if dtype == "bf16" else a)
        return out

    xs = [dev(a) for a in sample(0)]
    gs = [dev(a) for a in sample(1)]
    ys = [torch.empty_like(x) for x in xs]
    ms = [torch.empty((s[0], -(-s[1] // 32)), dtype=torch.int32, device="cuda") for s in shapes]
    gis = [torch.empty_like(x) for x in gs]

    def step():
        M.mxfp4_qdq_fwd_rows_batch(xs, ys, ms)
        M.mxfp4_ste_bwd_rows_batch(gs, ms, gis)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(4):
        xa, ga = sample(10 + rep), sample(20 + rep)
        for t, a in zip(xs, xa):
            t.copy_(dev(a))
        for t, a in zip(gs, ga):
            t.copy_(dev(a))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [host(t).copy() for t in ys + gis]
        junk = torch.randn(1 << 16, device="cuda").sum()   # eager work between replays
        step()                                              # the eager result on the same inputs
        torch.cuda.synchronize()
        want = [host(t) for t in ys + gis]
        for a, b in zip(got, want):
            assert np.array_equal(a, b)
        for i, a in enumerate(xa):
            yo, clip, _ = oracle.qdq_rows(a, 32)
            assert np.array_equal(got[i], yo)
            assert np.array_equal(got[len(shapes) + i], oracle.ste_bwd(ga[i], clip))
        assert torch.isfinite(junk)


def test_grouped_matmul_graph_replays_match_eager():
    """The row-split grouped matmul with more tiles than one round (its full
    rounds and its tail of 128 x 128 tiles: two launches per call) captured
    in a HIP graph: each replay, with new A codes copied into the captured
    buffer and eager work in between, equals the eager call bit for bit."""
    import mxfp4_fake_quantization_amd as M
    rng = np.random.default_rng(5)
    counts = [65536, 11254]                     # 300 tiles of 256 x 256 with N = 256
    Mr, N, K = sum(counts), 256, 256
    a = torch.empty((Mr, K), dtype=torch.uint8, device="cuda")
    sa = dev(rng.integers(120, 128, (Mr, K // 32)).astype(np.uint8))
    b = dev(rng.integers(0, 256, (2, N, K // 2)).astype(np.uint8))
    sb = dev(rng.integers(120, 128, (2, N, K // 32)).astype(np.uint8))
    gl = torch.tensor(counts, dtype=torch.int64, device="cuda")
    c = torch.empty((Mr, N), dtype=torch.bfloat16, device="cuda")
    c_eager = torch.empty_like(c)

    def codes(seed):
        return dev((np.random.default_rng(seed).integers(0, 256, (Mr, K)) & 0xBF).astype(np.uint8))

    a.copy_(codes(0))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        M.mxfp4_grouped_matmul(a, sa, b, sb, c, group_list=gl)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        M.mxfp4_grouped_matmul(a, sa, b, sb, c, group_list=gl)
    for rep in range(3):
        a.copy_(codes(1 + rep))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = host(c).copy()
        junk = torch.randn(1 << 16, device="cuda").sum()   # eager work between replays
        M.mxfp4_grouped_matmul(a, sa, b, sb, c_eager, group_list=gl)
        torch.cuda.synchronize()
        assert np.array_equal(got, host(c_eager))
        assert torch.isfinite(junk)
