"""Property fuzz of the whole layer on tiny shapes (hypothesis, derandomized).

Shapes: M and N in 1..300, K = 128..1024 (so every forward path for few rows,
few columns and small tiles is drawn: the one-launch forward up to 8 rows, the
few-row kernels, split-K and the tiled GEMM).  Activations mix random rows with
outlier columns, all-zero rows and the crafted corner-case rows (exact ties at
0.5 and 63.5, division against reciprocal, unit vectors, a wide exact spread,
tiny and huge scales); some examples scale every row by its own power of ten
between 1e-30 and 1e35 (row scales from far below 1 to far beyond 2^96, all
outputs normal and finite).  For every example:
  * the activation codes and scales and the int32 accumulators equal the
    oracle's, the forward equals its stages bit for bit, and its output is within
    the row tolerance of the oracle (and one bf16 ulp elementwise without bias);
  * when N is a multiple of 128, both input gradients match the oracle on every
    row.
CONVROT_FUZZ_EXAMPLES sets the number of examples (default 60) for a longer run
by hand; CONVROT_FUZZ_SEED, when set, replaces the fixed example sequence with
the one that seed draws.
"""
import os

import numpy as np
import pytest

import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
hyp = pytest.importorskip("hypothesis")
from hypothesis import HealthCheck, given, settings, strategies as st  # noqa: E402

from crafted import crafted_rows  # noqa: E402
from gpu_util import (Guarded, assert_exact, assert_fwd_elementwise, assert_rows_close,  # noqa: E402
                      bf16_to_dev, bits, guarded_workspace, host)


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


def _activations(M, K, seed, crafted_every, zero_every, magnitudes):
    x = wl.activations(M, K, max(1, wl.n_outliers(K)), base=seed)
    if magnitudes:
        f = wl.bf16_bits_to_f32(x).astype(np.float64)
        f *= 10.0 ** np.random.default_rng(seed).uniform(-30, 35, (M, 1))
        x = wl.f32_to_bf16_bits(f.astype(np.float32))
    special = crafted_rows(K)
    for m in range(M):
        if crafted_every and m % crafted_every == 0:
            x[m] = special[(m // crafted_every) % special.shape[0]]
        elif zero_every and m % zero_every == 1:
            x[m] = 0
    return x


_FUZZ_SEED = os.environ.get("CONVROT_FUZZ_SEED")


@settings(max_examples=int(os.environ.get("CONVROT_FUZZ_EXAMPLES", "60")), deadline=None,
          derandomize=_FUZZ_SEED is None, database=None,
          suppress_health_check=[HealthCheck.too_slow])
@given(M=st.integers(1, 300), N=st.integers(1, 300), kb=st.integers(1, 8),
       seed=st.integers(0, 1 << 20), crafted_every=st.sampled_from([0, 1, 3, 7]),
       zero_every=st.sampled_from([0, 2, 5]), magnitudes=st.booleans(), with_bias=st.booleans(),
       n128=st.booleans())
def test_tiny_layer_property(cr, orc, M, N, kb, seed, crafted_every, zero_every, magnitudes,
                             with_bias, n128):
    K = 128 * kb
    if n128:
        N = 128 * max(1, min(2, N // 128))
    print(f"fuzz M={M} N={N} K={K} seed={seed} crafted_every={crafted_every} "
          f"zero_every={zero_every} magnitudes={magnitudes} bias={with_bias}", flush=True)
    x = _activations(M, K, seed, crafted_every, zero_every, magnitudes)
    w = wl.normal_bf16((N, K), wl.SIGMA_W, seed, 1)
    bias_np = wl.normal_bf16((N,), 1.0, seed, 18) if with_bias else None
    bias = bf16_to_dev(bias_np) if with_bias else None
    qw, sw = cr.quantize_weight(bf16_to_dev(w))
    xd = bf16_to_dev(x)

    oqx, osx, _ = orc.rotate_quantize(x)
    oqw, osw, _ = orc.rotate_quantize(w)
    assert_exact(host(qw), oqw, "q_w")
    assert_exact(host(sw), osw, "s_w")
    qx, sx = cr.quantize_act(xd)
    assert_exact(host(qx), oqx, "q_x")
    assert_exact(host(sx), osx, "s_x")
    oacc = orc.gemm_i8_i32(oqx, oqw)
    assert_exact(host(cr.gemm_i8_i32(qx, qw, 0)), oacc, "acc")

    gy = Guarded((M, N), torch.bfloat16)
    gws = guarded_workspace(cr.workspace_bytes(cr.OP_LINEAR_FWD, M, N, K))
    y = cr.linear_fwd(xd, qw, sw, bias=bias, out=gy.t, workspace=gws.t)
    gy.check("y")
    gws.check("workspace")
    assert np.array_equal(bits(y), bits(cr.gemm_i8_bf16(qx, sx, qw, sw, bias=bias))), \
        "forward differs from its stages"
    oy = orc.dequant_epilogue(oacc, osx, osw, bias=bias_np)
    assert_rows_close(bits(y), oy, "y")
    if not with_bias:
        assert_fwd_elementwise(bits(y), oy, "y")

    if N % 128 == 0:
        dy = wl.normal_bf16((M, N), 1e-3, seed, 3)
        dyd = bf16_to_dev(dy)
        dx8 = cr.linear_bwd_dx(dyd, qw, sw, cr.BWD_INT8)
        dx16 = cr.linear_bwd_dx(dyd, qw, sw, cr.BWD_BF16)
        assert_rows_close(bits(dx8), orc.bwd_dx_int8(dy, oqw, osw)["dx"], "int8 dX")
        assert_rows_close(bits(dx16), orc.bwd_dx_bf16(dy, oqw, osw)["dx"], "bf16 dX")


if _FUZZ_SEED is not None:
    test_tiny_layer_property = hyp.seed(int(_FUZZ_SEED))(test_tiny_layer_property)
