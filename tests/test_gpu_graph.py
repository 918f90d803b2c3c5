"""The forward and the int8 input gradient captured in a HIP graph.

Every entry point is stream-ordered and allocates nothing, so a caller may
capture it (bench.py times the few-row forwards that way).  Each graph is
replayed several times with eager work on the same buffers in between, and every
replay must reproduce the eager result bit for bit: one case per forward path
(few-row kernel, its split form, each GEMM tile form, split-K, the one-launch
forward) and the int8 backward.
"""
import pytest

import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from gpu_util import bf16_to_dev  # noqa: E402


@pytest.fixture(scope="module")
def cr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import w8a8_rotated_int8_amd as cr
    cr.lib()
    return cr


def capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # first call outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


# few-row kernel, its split form, 128 x 64 tiles, 128 x 128 tiles with two and
# with four stages, split-K, 256 x 256 tiles, the one-launch forward
@pytest.mark.parametrize("M,K,N", [(77, 4096, 4096), (100, 8192, 1000), (300, 4096, 4096),
                                   (4096, 512, 2048), (1000, 1024, 4096), (300, 16384, 4096),
                                   (3072, 1024, 4096), (2, 4096, 4096)])
def test_forward_graph_replays(cr, M, K, N):
    print(f"graph forward M={M} K={K} N={N}", flush=True)
    x = bf16_to_dev(wl.activations(M, K, wl.n_outliers(K), base=5))
    qw, sw = cr.quantize_weight(bf16_to_dev(wl.packed_weight(5000 + N, 0, N, K)))
    ref = cr.linear_fwd(x, qw, sw)
    y = torch.empty_like(ref)
    ws = torch.empty(cr.workspace_bytes(cr.OP_LINEAR_FWD, M, N, K), dtype=torch.uint8,
                     device="cuda")
    g = capture(lambda: cr.linear_fwd(x, qw, sw, out=y, workspace=ws))
    for rep in range(3):
        y.zero_()
        ws.fill_(0x5a)                           # eager work on the captured buffers
        cr.linear_fwd(x, qw, sw)                 # and an eager call in between
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref), f"replay {rep} differs from the eager forward"


def test_int8_backward_graph_replays(cr):
    M, N, K = 256, 512, 384
    print(f"graph int8 dX M={M} N={N} K={K}", flush=True)
    dy = bf16_to_dev(wl.normal_bf16((M, N), 1e-3, 9, 3))
    qw, sw = cr.quantize_weight(bf16_to_dev(wl.packed_weight(5100, 0, N, K)))
    ref = cr.linear_bwd_dx(dy, qw, sw, cr.BWD_INT8)
    dx = torch.empty_like(ref)
    ws = torch.empty(cr.workspace_bytes(cr.OP_LINEAR_BWD_DX, M, N, K, cr.BWD_INT8),
                     dtype=torch.uint8, device="cuda")
    g = capture(lambda: cr.linear_bwd_dx(dy, qw, sw, cr.BWD_INT8, out=dx, workspace=ws))
    for rep in range(3):
        dx.zero_()
        ws.fill_(0x5a)
        cr.linear_bwd_dx(dy, qw, sw, cr.BWD_INT8)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(dx, ref), f"replay {rep} differs from the eager backward"
