"""Text-encoder shapes: one caption at a time (small, ragged M) and skinny
outputs (N = 32), as in the training guide's text-encoder quantization
(section 7.1, text encoder bullet).  With few 256 x 256 output tiles the
forward runs one of three paths:
  * the few-row kernel (M <= 128, N <= 8192, K <= 8192): 16 output columns per
    workgroup, the waves' int32 sums added in LDS; for K = 8192 and more than 32
    rows its split form, 64 columns and a 1 KB K-slice per workgroup into int32
    partials that one more launch sums and dequantizes;
  * the same kernel with the roles swapped for few output columns over many
    tokens (N <= 128, M >= 2048): 16 tokens per workgroup;
  * split-K: the contraction split into int32 partials that one more launch
    sums and dequantizes.

  * either forward equals the one-pass stages (quantize_act + the int8 GEMM
    with its dequantizing epilogue) bit for bit: integer sums are exact and the
    epilogue's fp32 operations are the same;
  * sampled rows match the oracle (1e-2 row tolerance; exact int32 sums).
"""
import numpy as np
import pytest

import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from gpu_util import (CANARY, Guarded, assert_exact, assert_fwd_elementwise,  # noqa: E402
                      assert_rows_close, bf16_to_dev, bits, guarded_workspace, host)


@pytest.fixture(scope="module")
def cr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import w8a8_rotated_int8_amd as cr
    cr.lib()
    return cr


# Row-tile counts 1..8 of the few-row kernel: ceil(M / 16) = 1 (1, 7, 16), 3 (33),
# 4 (64), 5 (77), 6 (90), 7 (100, 110) and 8 (128); the q_x-in-LDS variant for
# 3..8 tiles at K <= 4096 (three chunk buffers up to 6 tiles, two from 7 on).
SHAPES = [(1, 4096, 4096), (7, 4096, 4096), (77, 4096, 4096), (128, 4096, 4096),
          (33, 4096, 3000), (16, 8192, 2048), (100, 8192, 4096), (300, 4096, 4096),
          (64, 4096, 4096), (90, 4096, 2048), (110, 2048, 4096), (47, 1024, 2048),
          (77, 4096, 12288), (77, 12288, 4096), (77, 4096, 32), (4096, 4096, 32), (129, 512, 640),
          # few output columns over many tokens (the roles swapped): tile counts
          # ceil(N / 16) = 1, 3 (LDS), 7 (ragged, LDS) and 8 (LDS); K = 8192 direct
          (2048, 4096, 16), (4096, 2048, 48), (3000, 1024, 100), (2048, 4096, 128),
          (2500, 8192, 24),
          # few tokens and few or ragged output columns
          (1, 4096, 32), (16, 4096, 256), (77, 4096, 1000), (128, 1024, 64),
          # the split few-row form (K = 8192, 3 to 8 row tiles, ragged column groups)
          (33, 8192, 4096), (128, 8192, 8192), (100, 8192, 1000), (50, 8192, 4092),
          (32, 8192, 1024)]


@pytest.mark.parametrize("M,K,N", SHAPES)
def test_small_m_forward(cr, M, K, N):
    import oracle
    x = wl.activations(M, K, wl.n_outliers(K), base=0)
    w = wl.packed_weight(4000 + N % 997, 0, N, K)
    need = cr.workspace_bytes(cr.OP_LINEAR_FWD, M, N, K)
    one_pass = ((M * K + 255) // 256) * 256 + ((4 * M + 255) // 256) * 256
    print(f"M={M} K={K} N={N}: workspace {need} B ({'split' if need > one_pass else 'one pass'})",
          flush=True)
    qw, sw = cr.quantize_weight(bf16_to_dev(w))
    xd = bf16_to_dev(x)
    gy, gws = Guarded((M, N), torch.bfloat16), guarded_workspace(need)
    y = cr.linear_fwd(xd, qw, sw, out=gy.t, workspace=gws.t)
    gy.check("y")
    gws.check("workspace (q_x, s_x, partials)")
    qx, sx = cr.quantize_act(xd)
    y1 = cr.gemm_i8_bf16(qx, sx, qw, sw)
    assert torch.equal(y, y1), "split forward differs from the one-pass stages"
    g = np.random.default_rng(71 + M)
    rows = np.unique(np.concatenate([[0, M - 1], g.choice(M, min(M, 6), replace=False)]))
    oqx, osx, _ = oracle.rotate_quantize(x[rows])
    oqw, osw, _ = oracle.rotate_quantize(w)
    assert_exact(host(qx)[rows], oqx, "q_x (sampled rows)")
    oacc = oracle.gemm_i8_i32(oqx, oqw)
    assert_exact(host(cr.gemm_i8_i32(qx, qw, 0))[rows], oacc, "acc (sampled rows)")
    oy = oracle.dequant_epilogue(oacc, osx, osw)
    e = assert_rows_close(bits(y)[rows], oy, "y (sampled rows)")
    assert_fwd_elementwise(bits(y)[rows], oy, "y (sampled rows)")
    print(f"  max row relerr {e:.2e}", flush=True)


@pytest.mark.parametrize("M,K,N", [(77, 4096, 4096), (4096, 4096, 32), (2048, 2048, 100),
                                   (77, 8192, 2048)])
def test_small_m_with_bias(cr, M, K, N):
    x = wl.activations(M, K, wl.n_outliers(K), base=1)
    w = wl.packed_weight(4100, 1, N, K)
    bias = bf16_to_dev(wl.normal_bf16((N,), 1.0, 1, 18))
    qw, sw = cr.quantize_weight(bf16_to_dev(w))
    xd = bf16_to_dev(x)
    y = cr.linear_fwd(xd, qw, sw, bias=bias)
    qx, sx = cr.quantize_act(xd)
    assert torch.equal(y, cr.gemm_i8_bf16(qx, sx, qw, sw, bias=bias))


# The one-launch forward of very few rows: every workgroup rotates and
# quantizes x's rows itself, in LDS, and runs the few-row contraction (at most
# 8 / ceil(K / 2048) rows).  Shapes: one wave per row (K <= 2048; power-of-two
# and other block counts, up to 8 rows), two (K = 4096, up to 4 rows), three
# (K = 4224 and 6144: 2 rows, two waves without a row) and four (K = 8192, 2
# rows); ragged and skinny N.
FUSED = [(1, 128, 4096), (8, 128, 40), (3, 384, 1000), (8, 1152, 4096), (5, 2048, 2000),
         (8, 2048, 16), (1, 4096, 4096), (2, 4096, 4096), (4, 4096, 4096), (3, 4096, 8192),
         (1, 4224, 4096), (2, 6144, 1000), (2, 8192, 4096), (1, 8192, 8)]


@pytest.mark.parametrize("with_bias", [False, True])
@pytest.mark.parametrize("M,K,N", FUSED)
def test_fused_few_row_forward(cr, M, K, N, with_bias):
    import oracle
    print(f"fused forward M={M} K={K} N={N} bias={with_bias}", flush=True)
    x = wl.activations(M, K, wl.n_outliers(K), base=2)
    w = wl.packed_weight(4200 + N % 997, 2, N, K)
    bias_np = wl.normal_bf16((N,), 1.0, 2, 19) if with_bias else None
    bias = bf16_to_dev(bias_np) if with_bias else None
    qw, sw = cr.quantize_weight(bf16_to_dev(w))
    xd = bf16_to_dev(x)
    gy = Guarded((M, N), torch.bfloat16)
    gws = guarded_workspace(cr.workspace_bytes(cr.OP_LINEAR_FWD, M, N, K))
    y = cr.linear_fwd(xd, qw, sw, bias=bias, out=gy.t, workspace=gws.t)
    gy.check("y")
    gws.check("workspace")
    # q_x and s_x never leave LDS: the workspace still holds the canary (the
    # two-launch forward writes q_x there), so this is the one-launch path
    assert bool((gws.t == CANARY).all()), "the workspace was written: not the one-launch forward"
    qx, sx = cr.quantize_act(xd)
    y1 = cr.gemm_i8_bf16(qx, sx, qw, sw, bias=bias)
    assert np.array_equal(bits(y), bits(y1)), "one-launch forward differs from the two launches"
    oqx, osx, _ = oracle.rotate_quantize(x)
    oqw, osw, _ = oracle.rotate_quantize(w)
    assert_exact(host(qx), oqx, "q_x")
    oy = oracle.dequant_epilogue(oracle.gemm_i8_i32(oqx, oqw), osx, osw, bias=bias_np)
    e = assert_rows_close(bits(y), oy, "y")
    if not with_bias:  # the one-ulp bound is for the product alone (a bias can cancel it)
        assert_fwd_elementwise(bits(y), oy, "y")
    print(f"  max row relerr {e:.2e}", flush=True)


@pytest.mark.parametrize("M,K", [(2, 4096), (8, 1024), (2, 8192)])
def test_fused_few_row_forward_nonfinite_row(cr, M, K):
    # a NaN or infinite activation gives its row the NaN scale, in the fused
    # quantization as in the activation quantizer: a NaN output row, the other
    # rows unchanged, and the two-launch forward's bits
    N = 1000
    x = wl.activations(M, K, wl.n_outliers(K), base=3)
    w = wl.packed_weight(4300, 3, N, K)
    qw, sw = cr.quantize_weight(bf16_to_dev(w))
    y0 = bits(cr.linear_fwd(bf16_to_dev(x), qw, sw))
    xb = x.copy()
    xb[M - 1, 5] = 0x7FC0                     # NaN
    if M > 2:
        xb[1, K - 1] = 0xFF80                 # -inf
    xd = bf16_to_dev(xb)
    y = bits(cr.linear_fwd(xd, qw, sw))
    qx, sx = cr.quantize_act(xd)
    assert np.array_equal(y, bits(cr.gemm_i8_bf16(qx, sx, qw, sw)))
    bad = [M - 1] + ([1] if M > 2 else [])
    yf = wl.bf16_bits_to_f32(y)
    for r in bad:
        assert np.isnan(yf[r]).all(), f"row {r} should be NaN"
    keep = np.setdiff1d(np.arange(M), bad)
    assert np.array_equal(y[keep], y0[keep])
