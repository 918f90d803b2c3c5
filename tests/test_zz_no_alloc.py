"""The allocation-free forward (convrot_linear_fwd_noalloc) against the
workspace forward (convrot_linear_fwd), through the C ABI.

Both run the same kernels; the allocation-free one keeps q_x, s_x and any
split-K partials in the library's static per-GPU scratch.  Outputs must be equal
bit for bit on consecutive calls of decreasing size (so that the second call
finds the first call's contents in the scratch), across the forward's paths
(tiled GEMM, split-K, few-row kernel), with canary bands around the outputs.
Oversized calls are refused with CONVROT_ESCRATCH and leave the output alone.
"""
import numpy as np
import pytest

import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from gpu_util import Guarded, bf16_to_dev  # noqa: E402


@pytest.fixture(scope="module")
def cr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import w8a8_rotated_int8_amd as cr
    cr.lib()
    return cr


def _layer(cr, M, K, N, base):
    x = bf16_to_dev(wl.activations(M, K, wl.n_outliers(K), base=base))
    qw, sw = cr.quantize_weight(bf16_to_dev(wl.packed_weight(base, base, N, K)))
    return x, qw, sw


@pytest.mark.parametrize("shapes", [
    [(4096, 4096, 4096), (300, 16384, 4096)],    # 256 x 256 tiles, then split-K
    [(1000, 4096, 4096), (300, 4096, 4096)],     # 128 x 128 tiles, then 128 x 64 tiles
    [(20480, 4096, 4096), (77, 4096, 4096)],     # the packed stream, then the few-row kernel
    [(4096, 16384, 4096), (2048, 4096, 32)],     # MLP down input, then skinny outputs
    [(4096, 4096, 4096), (2, 4096, 4096)],       # tiled GEMM, then the one-launch few-row forward
])
def test_noalloc_matches_workspace_forward(cr, shapes):
    for i, (M, K, N) in enumerate(shapes):
        print(f"noalloc call {i}: M={M} K={K} N={N}", flush=True)
        x, qw, sw = _layer(cr, M, K, N, base=M + N + i)
        ref = cr.linear_fwd(x, qw, sw)
        gy = Guarded((M, N), torch.bfloat16)
        y = cr.linear_fwd_noalloc(x, qw, sw, out=gy.t)
        gy.check("noalloc y")
        assert torch.equal(y, ref), f"call {i} differs from the workspace forward"


def test_noalloc_with_bias_and_repeat(cr):
    M, K, N = 1000, 2048, 640
    x, qw, sw = _layer(cr, M, K, N, base=5)
    bias = bf16_to_dev(wl.normal_bf16((N,), 1.0, 5, 18))
    ref = cr.linear_fwd(x, qw, sw, bias=bias)
    for _ in range(2):
        assert torch.equal(cr.linear_fwd_noalloc(x, qw, sw, bias=bias), ref)


def test_noalloc_refuses_oversized_calls(cr):
    M, K, N = 32768, 4096, 128
    x = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    qw = torch.zeros((N, K), dtype=torch.int8, device="cuda")
    sw = torch.ones((N,), dtype=torch.float32, device="cuda")
    y = torch.full((M, N), 3.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(cr.ConvRotError) as ei:
        cr.linear_fwd_noalloc(x, qw, sw, out=y)
    assert ei.value.status == -6
    torch.cuda.synchronize()
    assert bool((y == 3.0).all())
    # the entry point still works afterwards
    x2, qw2, sw2 = _layer(cr, 64, 256, 256, base=9)
    assert torch.equal(cr.linear_fwd_noalloc(x2, qw2, sw2), cr.linear_fwd(x2, qw2, sw2))
