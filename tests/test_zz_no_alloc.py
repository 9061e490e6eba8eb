"""bitlinear_forward_noalloc (the entry point for callers that cannot
allocate) against bitlinear_forward, called through the C ABI: two calls in a
row on shapes whose plan splits K over workgroups (so the library's scratch
carries the split-K slots), the second smaller, then shapes that need no
scratch, a shape whose slots would not fit, and a HIP graph replayed with
eager work between the replays."""
import numpy as np
import pytest

from datagen import random_case
from gpu_util import dev, host, log, x_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_gemm_int8_amd as B
    return B


def _case(B, m, n, k, seed):
    w, x = random_case(seed, m, n, k, x_kind="t3")
    xd, _ = x_device(x, "bf16")
    packed, gamma = B.pack_weights(dev(w))
    xq, s = B.quant_act(xd)
    return xq, s, packed, gamma


def _both(B, m, n, k, relu2, seed):
    """(y, acc) from bitlinear_forward and from bitlinear_forward_noalloc."""
    import torch
    xq, s, packed, gamma = _case(B, m, n, k, seed)
    y0, a0 = B.forward(xq, s, packed, gamma, n, k, relu2=relu2, out_dtype=torch.bfloat16,
                       acc_out=True, workspace=B.Workspace())
    a1 = torch.empty((m, n), dtype=torch.int32, device="cuda")
    y1 = B.forward_noalloc(xq, s, packed, gamma, n, k, relu2=relu2, out_dtype=torch.bfloat16,
                           acc_out=a1)
    return (host(y0), host(a0)), (host(y1), host(a1))


def _same(r0, r1, where):
    np.testing.assert_array_equal(r1[1], r0[1], err_msg=f"{where} acc")
    np.testing.assert_array_equal(r1[0], r0[0], err_msg=f"{where} y")


# (m, n, k, relu2): split-K plans of the dot4 GEMV (fewer than 1024 rows, or
# rows too long for the streaming kernel's LDS), the second call of each
# pair smaller than the first
SPLIT_PAIRS = [((1, 960, 16384, False), (1, 300, 12288, True)),
               ((2, 8192, 40000, True), (2, 640, 20000, False))]


@pytest.mark.parametrize("first,second", SPLIT_PAIRS)
def test_noalloc_matches_forward_two_calls(B, first, second):
    for i, (m, n, k, relu2) in enumerate((first, second)):
        assert B.forward_workspace_bytes(m, n, k) > 0          # the scratch is used
        log(f"noalloc m={m} n={n} k={k} call {i}")
        r0, r1 = _both(B, m, n, k, relu2, 6100 + 13 * i + n)
        _same(r0, r1, f"call {i} ({m}, {n}, {k})")


@pytest.mark.parametrize("m,n,k", [(1, 2560, 2560), (1, 8192, 28672), (16, 8192, 8192),
                                   (300, 2560, 6912)])
def test_noalloc_without_split(B, m, n, k):
    assert B.forward_workspace_bytes(m, n, k) == 0
    log(f"noalloc m={m} n={n} k={k}")
    r0, r1 = _both(B, m, n, k, False, 6200 + m)
    _same(r0, r1, f"({m}, {n}, {k})")


def test_noalloc_refuses_oversized_scratch(B):
    # 2 tokens, K long enough that the x~ slice forces a split over workgroups
    # of a matrix with >= 256 row blocks: more slots than the scratch holds
    m, n, k = 2, 16448, 65536
    need = B.forward_workspace_bytes(m, n, k)
    assert need > B.BL_NOALLOC_SCRATCH_BYTES
    import torch
    xq = torch.zeros((m, k), dtype=torch.int8, device="cuda")
    s = torch.ones(m, dtype=torch.float32, device="cuda")
    packed = torch.zeros(B.packed_bytes(64, k), dtype=torch.uint8, device="cuda")   # never read
    gamma = torch.ones(1, dtype=torch.float32, device="cuda")
    y = torch.empty((m, n), dtype=torch.float32, device="cuda")
    st = B.lib.bitlinear_forward_noalloc(xq.data_ptr(), s.data_ptr(), packed.data_ptr(),
                                         gamma.data_ptr(), m, n, k, 0, 0, y.data_ptr(), None,
                                         B._stream())
    assert st == 4                                            # BL_ERR_WORKSPACE, nothing launched


def test_noalloc_graph_replays(B):
    """Captured in a graph, replayed three times with eager calls of the same
    entry point (other shapes, split plans) between the replays: every replay
    gives the eager result."""
    import torch
    m, n, k = 1, 960, 16384
    assert B.forward_workspace_bytes(m, n, k) > 0
    xq, s, packed, gamma = _case(B, m, n, k, 6300)
    ref = torch.empty((m, n), dtype=torch.int32, device="cuda")
    yref = B.forward_noalloc(xq, s, packed, gamma, n, k, acc_out=ref)
    acc = torch.zeros_like(ref)
    y = torch.empty_like(yref)
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=st):
        B.forward_noalloc(xq, s, packed, gamma, n, k, y=y, acc_out=acc, stream=st)
    torch.cuda.synchronize()
    other = _case(B, 2, 640, 20000, 6301)
    for r in range(3):
        acc.zero_()
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(acc, ref), f"replay {r}"
        assert torch.equal(y, yref), f"replay {r}"
        B.forward_noalloc(*other, 640, 20000)             # eager work between replays
        torch.cuda.synchronize()
