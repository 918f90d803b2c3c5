"""Seeded sweep of layer shapes across every dispatch boundary of the forward and
both input gradients.

The forward picks among the tiled GEMM (256 x 256, 128 x 128 or 128 x 64 tiles), split-K,
the few-row kernel (either role) and, for very few rows, the one-launch forward
from M, N and K; the shapes here are drawn around those boundaries (M near 128
and 2048, N near 128, 2048 and 8192, K from 128 to 12288, ragged sizes, either
side of the one-launch row limit and of the tile-count limits of the small
tiles).
For each shape:
  * the forward equals the one-pass stages (quantize_act, then the int8 GEMM
    with its dequantizing epilogue) bit for bit, whichever path it took;
  * the forward's rows (all of them up to 2^28 multiply-adds, else three
    sampled rows) and three sampled rows of both input gradients match the
    oracle: exact codes, scales and int32 sums, outputs within the 1e-2 row
    tolerance, and the forward within one bf16 ulp element by element.
CONVROT_SWEEP_EXTRA=n adds n seeded random shapes (CONVROT_SWEEP_SEED, default
777) for a wider run by hand; the default run is the fixed list.
"""
import os

import numpy as np
import pytest

import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from gpu_util import (Guarded, assert_exact, assert_fwd_elementwise, assert_rows_close,  # noqa: E402
                      bf16_to_dev, bits, guarded_workspace, host)


def _shapes():
    g = np.random.default_rng(20261202)
    picks = []
    Ms = [1, 5, 64, 127, 128, 129, 300, 1000, 2047, 2048, 2500, 4096]
    Ns = [8, 24, 100, 128, 130, 640, 2000, 2048, 4100, 8192, 8200, 12288]
    Ks = [128, 256, 640, 1024, 2048, 4096, 8192, 12288]
    for _ in range(28):
        M, N, K = int(g.choice(Ms)), int(g.choice(Ns)), int(g.choice(Ks))
        # keep each case to about a second, the oracle's full-weight quantization included
        while N * K > 1 << 25 or M * N * K > 1 << 35:
            K = max(128, K // 2)
            if N * K > 1 << 25 or M * N * K > 1 << 35:
                N = max(8, N // 2)
        picks.append((M, N, K))
    # few output columns over many tokens (the swapped few-row path)
    picks += [(2048, 100, 1024), (3000, 24, 2048), (4096, 128, 512)]
    # either side of the one-launch forward's row limit, 8 / ceil(K / 2048) rows
    picks += [(8, 640, 2048), (9, 640, 2048), (4, 1000, 4096), (5, 1000, 4096),
              (2, 130, 6144), (3, 130, 6144), (2, 2000, 8192), (3, 2000, 8192)]
    # the one-pass GEMM's tile choice: 128 x 64 tiles up to 256 tiles, 128 x 128
    # tiles with four stages up to 256 tiles, with two stages up to 512, then
    # 256 x 256; ragged edges, and N below 4 (no split-K)
    picks += [(257, 1000, 640), (1024, 4096, 1024), (1025, 4096, 1024), (2047, 4096, 1024),
              (2049, 4096, 1024), (1500, 4100, 512), (300, 3, 1024), (700, 1, 384),
              (512, 4096, 1024), (513, 4096, 1024), (65, 8200, 256), (300, 32, 2048),
              (300, 4096, 4096), (1000, 4096, 4096), (1500, 4096, 4096)]
    picks += _extra_shapes(int(os.environ.get("CONVROT_SWEEP_EXTRA", "0")),
                           int(os.environ.get("CONVROT_SWEEP_SEED", "777")))
    return sorted(set(picks))


def _extra_shapes(n, seed):
    """Opt-in wider sweep (CONVROT_SWEEP_EXTRA shapes, seed CONVROT_SWEEP_SEED):
    a third of the shapes with at most 8 rows (the one-launch and few-row
    forwards at many K), any N up to 9000, any multiple of 128 up to 12288 for K,
    under the same per-case size bounds."""
    g = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        r = g.random()
        M = (int(g.integers(1, 9)) if r < 0.35 else
             int(g.integers(9, 300)) if r < 0.6 else int(g.integers(300, 5000)))
        N = int(g.integers(1, 9000)) if g.random() < 0.7 else int(128 * g.integers(1, 70))
        K = int(128 * g.integers(1, 97))
        while N * K > 1 << 25 or M * N * K > 1 << 35:
            if K > 128 and g.random() < 0.5:
                K = max(128, (K // 256) * 128)
            else:
                N = max(1, N // 2)
        out.append((M, N, K))
    return out


@pytest.fixture(scope="module")
def cr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import w8a8_rotated_int8_amd as cr
    cr.lib()
    return cr


@pytest.fixture(scope="module")
def orc():
    import oracle
    oracle.lib()
    return oracle


@pytest.mark.parametrize("M,N,K", _shapes())
def test_shape(cr, orc, M, N, K):
    print(f"sweep M={M} N={N} K={K}", flush=True)
    base = M + 7 * N + 13 * K
    x = wl.activations(M, K, max(1, wl.n_outliers(K)), base=base)
    w = wl.packed_weight(base % 997, base, N, K)
    qw, sw = cr.quantize_weight(bf16_to_dev(w))
    xd = bf16_to_dev(x)
    gy = Guarded((M, N), torch.bfloat16)
    gws = guarded_workspace(cr.workspace_bytes(cr.OP_LINEAR_FWD, M, N, K))
    y = cr.linear_fwd(xd, qw, sw, out=gy.t, workspace=gws.t)
    gy.check("y")
    gws.check("workspace")
    qx, sx = cr.quantize_act(xd)
    assert torch.equal(y, cr.gemm_i8_bf16(qx, sx, qw, sw)), "forward differs from its stages"

    # every forward row where the oracle's GEMM stays small, else three
    # sampled rows (the gradients: the sampled rows)
    sampled = np.unique(np.array([0, M - 1, (M * 5) // 7]))
    rows = np.arange(M) if M * N * K <= 1 << 28 else sampled
    oqw, osw, _ = orc.rotate_quantize(w)
    assert_exact(host(qw), oqw, "q_w")
    assert_exact(host(sw), osw, "s_w")
    oqx, osx, _ = orc.rotate_quantize(x[rows])
    assert_exact(host(qx)[rows], oqx, "q_x rows")
    assert_exact(host(sx)[rows], osx, "s_x rows")
    oacc = orc.gemm_i8_i32(oqx, oqw)
    oy = orc.dequant_epilogue(oacc, osx, osw)
    assert_rows_close(bits(y)[rows], oy, "y rows")
    assert_fwd_elementwise(bits(y)[rows], oy, "y rows")

    if N % 128 == 0:
        dy = wl.normal_bf16((M, N), 1e-3, base, 3)
        dyd = bf16_to_dev(dy)
        gd8, gd16 = Guarded((M, K), torch.bfloat16), Guarded((M, K), torch.bfloat16)
        dx8 = cr.linear_bwd_dx(dyd, qw, sw, cr.BWD_INT8, out=gd8.t)
        dx16 = cr.linear_bwd_dx(dyd, qw, sw, cr.BWD_BF16, out=gd16.t)
        gd8.check("int8 dX")
        gd16.check("bf16 dX")
        assert_rows_close(bits(dx8)[sampled], orc.bwd_dx_int8(dy[sampled], oqw, osw)["dx"],
                          "int8 dX rows")
        assert_rows_close(bits(dx16)[sampled], orc.bwd_dx_bf16(dy[sampled], oqw, osw)["dx"],
                          "bf16 dX rows")
