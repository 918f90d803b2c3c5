"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Codes, scales and int32 accumulators must match bit for bit; bf16 outputs must
be within 1e-2 of the oracle per row (max abs error / max abs reference).
Small cases are compared element by element in full; the full-size workloads
are compared in full where the oracle is fast (quantizers) and on seeded
sampled rows where it is not (GEMM outputs).
"""
import numpy as np
import pytest

import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


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


from crafted import crafted_rows, nonfinite_fold_rows, nonfinite_rows, tiny_fold_rows  # noqa: E402
from gpu_util import (Guarded, assert_exact, assert_fwd_elementwise, assert_rows_close,  # noqa: E402
                      bf16_to_dev, bits, guarded_workspace, host, to_dev)


def say(*a):
    print(*a, flush=True)


# --------------------------------------------------------------------------
# Quantizer (weights, activations, embedding chunks)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("M,K", [(1, 128), (3, 256), (64, 256), (301, 384), (40, 512),
                                 (37, 1024), (19, 1152), (23, 1920), (31, 2048), (9, 2176),
                                 (97, 4096), (33, 4224), (16, 12288), (24, 16384), (5, 32768)])
def test_quantize_act_exact(cr, orc, M, K):
    say(f"quantize_act M={M} K={K}")
    x = wl.activations(M, K, max(1, wl.n_outliers(K)), base=M + K)
    x = np.concatenate([x, crafted_rows(K)])
    gq, gs = Guarded(x.shape, torch.int8), Guarded((x.shape[0],), torch.float32)
    q, s = cr.quantize_act(bf16_to_dev(x), out=(gq.t, gs.t))
    gq.check("codes")
    gs.check("scales")
    oq, os_, bad = orc.rotate_quantize(x)
    assert bad == 0
    assert_exact(host(s), os_, "scales")
    assert_exact(host(q), oq, "codes")


NAN_BITS = 0x7FC00000


@pytest.mark.parametrize("K", [128, 256, 4096, 4224, 16384])
def test_quantize_nonfinite_rows(cr, orc, K):
    # rows with a NaN or infinite rotated value (non-finite inputs, an inf - inf
    # block, an fp32 overflow of the rotation): NaN scale and zero codes on
    # every quantizer path, bit for bit with the oracle; ordinary rows around
    # them are unaffected (short rows share a wave with their neighbours)
    say(f"quantize nonfinite rows K={K}")
    x = np.concatenate([wl.activations(37, K, max(1, wl.n_outliers(K)), base=K),
                        nonfinite_rows(K, K), wl.activations(5, K, 1, base=K + 1)])
    oq, os_, _ = orc.rotate_quantize(x)
    assert (os_[37:43].view(np.uint32) == NAN_BITS).all() and not oq[37:43].any()
    for name, fn in (("act", cr.quantize_act), ("weight", cr.quantize_weight)):
        q, s = fn(bf16_to_dev(x))
        assert_exact(host(s), os_, f"{name} scales")
        assert_exact(host(q), oq, f"{name} codes")


def test_quantize_nonfinite_rows_row_kernel(cr, orc):
    # the 4096-wide row kernel (8192 rows and more, activations and chunked
    # weights): crafted rows at the start, middle and end of the batch
    say("quantize nonfinite rows, 8192 x 4096 row kernel")
    K, M = 4096, 8192
    x = np.zeros((M, K), np.uint16)
    bad = nonfinite_rows(K, 3)
    picks = [0, 1, 4095, 4096, M - 8, M - 1]
    for i, r in enumerate(picks):
        x[r] = bad[i % bad.shape[0]]
    x[100] = bad[6]  # an ordinary row
    rows = picks + [100]
    oq, os_, _ = orc.rotate_quantize(x[rows])
    for name, fn in (("act", lambda t: cr.quantize_act(t)),
                     ("weight", lambda t: cr.quantize_weight(t, chunk_rows=M))):
        q, s = fn(bf16_to_dev(x))
        assert_exact(host(s)[rows], os_, f"{name} scales")
        assert_exact(host(q)[rows], oq, f"{name} codes")


@pytest.mark.parametrize("N", [256, 2048, 4224])
def test_bwd_quant_dy_nonfinite_rows(cr, orc, N):
    say(f"bwd_quant_dy nonfinite rows N={N}")
    dy, sw = nonfinite_fold_rows(N, N)
    qg, sg = cr.bwd_quant_dy(bf16_to_dev(dy), torch.from_numpy(sw).cuda())
    oqg, osg = orc.bwd_quant_dy(dy, sw)
    assert (osg[:4].view(np.uint32) == NAN_BITS).all() and np.isfinite(osg[4])
    assert_exact(host(sg), osg, "s_g")
    assert_exact(host(qg), oqg, "q_g")


def test_forward_nonfinite_row_gives_nan_output_row(cr):
    # a NaN activation row comes out of the forward as a NaN output row; the
    # other rows are the same as without it
    say("forward with a nonfinite activation row")
    t = wl.tiny(0)
    x = t["x"].copy()
    x[3, 17] = 0x7FC0
    qw, sw = cr.quantize_weight(bf16_to_dev(t["w"]))
    y = bits(cr.linear_fwd(bf16_to_dev(x), qw, sw))
    y0 = bits(cr.linear_fwd(bf16_to_dev(t["x"]), qw, sw))
    yf = wl.bf16_bits_to_f32(y)
    assert np.isnan(yf[3]).all()
    keep = np.arange(x.shape[0]) != 3
    assert np.array_equal(y[keep], y0[keep])


def _huge_rows(M, K, base):
    """Activation rows whose scales lie beyond 2^96 (values ~1e33 .. 3e36, where
    fl32(acc * s_x) would leave the fp32 range although the output does not),
    mixed with ordinary rows and the crafted corner rows."""
    x = wl.activations(M, K, max(1, wl.n_outliers(K)), base=base)
    f = wl.bf16_bits_to_f32(x).astype(np.float64)
    g = np.random.default_rng(base)
    for m in range(0, M, 2):
        f[m] *= 10.0 ** g.uniform(33, 35.5)
    x = wl.f32_to_bf16_bits(f.astype(np.float32))
    return np.concatenate([x, crafted_rows(K)])


@pytest.mark.parametrize("M,K,N", [(300, 512, 640), (77, 4096, 1000), (2, 4096, 4096),
                                   (4096, 256, 300), (2048, 1024, 32), (60, 8192, 256)])
def test_forward_huge_activation_scales(cr, orc, M, K, N):
    # split-K, the few-row kernels, the one-launch forward, the tiled GEMM and
    # the swapped roles: every path gives the oracle's finite outputs where the
    # plain fp32 chain would overflow, and the paths agree bit for bit
    say(f"forward with row scales beyond 2^96 M={M} K={K} N={N}")
    x = _huge_rows(M, K, 500 + M)
    w = wl.packed_weight(4400 + N % 97, 4, N, K)
    qw, sw = cr.quantize_weight(bf16_to_dev(w))
    xd = bf16_to_dev(x)
    y = cr.linear_fwd(xd, qw, sw)
    qx, sx = cr.quantize_act(xd)
    assert np.array_equal(bits(y), bits(cr.gemm_i8_bf16(qx, sx, qw, sw))), "paths differ"
    assert float(host(sx).max()) > 2.0 ** 96
    rows = np.unique(np.concatenate([np.arange(0, x.shape[0], max(1, x.shape[0] // 40)),
                                     np.arange(x.shape[0] - 11, x.shape[0])]))
    oqx, osx, _ = orc.rotate_quantize(x[rows])
    oqw, osw, _ = orc.rotate_quantize(w)
    assert_exact(host(qx)[rows], oqx, "q_x rows")
    oy = orc.dequant_epilogue(orc.gemm_i8_i32(oqx, oqw), osx, osw)
    yb = bits(y)[rows]
    assert np.isfinite(wl.bf16_bits_to_f32(oy)).all()
    assert np.isfinite(wl.bf16_bits_to_f32(yb)).all()
    assert_rows_close(yb, oy, "y rows")
    assert_fwd_elementwise(yb, oy, "y rows")


def test_lora_forward_huge_activation_scales(cr, orc):
    M, K, N, R = 130, 512, 384, 16
    say("LoRA forward with row scales beyond 2^96")
    x = _huge_rows(M, K, 77)
    w = wl.packed_weight(4500, 5, N, K)
    lw = wl.lora_weights(K, N, R, 5)
    qw, sw = cr.quantize_weight(bf16_to_dev(w))
    xd, ad, bd = bf16_to_dev(x), bf16_to_dev(lw["a"]), bf16_to_dev(lw["b"])
    y = cr.linear_fwd_lora(xd, qw, sw, ad, bd, 0.5)
    oqx, osx, _ = orc.rotate_quantize(x)
    oqw, osw, _ = orc.rotate_quantize(w)
    ref = orc.lora_epilogue(orc.gemm_i8_i32(oqx, oqw), osx, osw, bits(cr.lora_down(xd, ad)), lw["b"], 0.5)
    assert np.isfinite(wl.bf16_bits_to_f32(bits(y))).all()
    assert_rows_close(bits(y), ref, "y")


@pytest.mark.parametrize("M,N,K", [(64, 256, 384), (37, 4096, 512)])
def test_bwd_int8_huge_gradient_scales(cr, orc, M, N, K):
    # dY rows whose folded scales s_g lie beyond 2^96: the inverse rotation's
    # fp32 sums stay in range and dX matches the oracle
    say(f"int8 dX with s_g beyond 2^96 M={M} N={N} K={K}")
    dy = wl.normal_bf16((M, N), 1e-3, M, 3)
    f = wl.bf16_bits_to_f32(dy).astype(np.float64)
    f[::3] *= 1e38
    dy = wl.f32_to_bf16_bits(f.astype(np.float32))
    w = wl.normal_bf16((N, K), wl.SIGMA_W, M, 1)
    e = _bwd_int8(cr, orc, dy, w)
    print(f"  max row relerr {e:.2e}", flush=True)


def test_quantize_weight_tiny_and_chunked(cr, orc):
    t = wl.tiny(0)
    say("quantize_weight tiny")
    q, s = cr.quantize_weight(bf16_to_dev(t["w"]))
    oq, os_, _ = orc.rotate_quantize(t["w"])
    assert_exact(host(q), oq, "codes")
    assert_exact(host(s), os_, "scales")
    for chunk in (1, 7, 100, 256):
        qc, sc = cr.quantize_weight(bf16_to_dev(t["w"]), chunk_rows=chunk)
        assert_exact(host(qc), oq, f"codes chunk={chunk}")
        assert_exact(host(sc), os_, f"scales chunk={chunk}")


def test_quantize_is_deterministic(cr):
    x = bf16_to_dev(wl.activations(512, 4096, 41, base=4))
    q1, s1 = cr.quantize_act(x)
    q2, s2 = cr.quantize_act(x)
    assert torch.equal(q1, q2) and torch.equal(s1, s2)


# --------------------------------------------------------------------------
# int32 contraction
# --------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (64, 256, 256), (300, 200, 384), (257, 513, 1024),
                                   (512, 512, 4096), (33, 700, 16384)])
def test_gemm_i32_exact(cr, orc, M, N, K):
    say(f"gemm_i8_i32 b_layout=0 M={M} N={N} K={K}")
    g = np.random.default_rng(M * 7 + N)
    a = g.integers(-127, 128, (M, K), dtype=np.int8)
    b = g.integers(-127, 128, (N, K), dtype=np.int8)
    acc = cr.gemm_i8_i32(to_dev(a), to_dev(b), 0)
    assert_exact(host(acc), orc.gemm_i8_i32(a, b), "acc")


def test_gemm_i32_extreme_values(cr, orc):
    M, N, K = 64, 256, 16384
    a = np.full((M, K), -127, np.int8)
    b = np.full((N, K), -127, np.int8)
    b[1::2] = 127
    acc = cr.gemm_i8_i32(to_dev(a), to_dev(b), 0)
    assert_exact(host(acc), orc.gemm_i8_i32(a, b), "acc")


@pytest.mark.parametrize("M,N,K", [(64, 256, 256), (1, 128, 128), (300, 384, 640), (129, 4096, 512)])
def test_gemm_i32_rows_of_b_exact(cr, orc, M, N, K):
    # acc[m][n] = sum_k a[m][k] b[k][n]  (the int8 input-gradient contraction)
    say(f"gemm_i8_i32 b_layout=1 M={M} N={N} K={K}")
    g = np.random.default_rng(M + N + K)
    a = g.integers(-127, 128, (M, K), dtype=np.int8)
    b = g.integers(-127, 128, (K, N), dtype=np.int8)
    acc = cr.gemm_i8_i32(to_dev(a), to_dev(b), 1)
    assert_exact(host(acc), orc.gemm_i8_i32_rows_of_b(a, b), "acc")


# --------------------------------------------------------------------------
# Forward
# --------------------------------------------------------------------------

def _fwd_case(cr, orc, x, w, bias=None, rows=None):
    qw, sw = cr.quantize_weight(bf16_to_dev(w))
    M, N = x.shape[0], w.shape[0]
    gy = Guarded((M, N), torch.bfloat16)
    gws = guarded_workspace(cr.workspace_bytes(cr.OP_LINEAR_FWD, M, N, x.shape[1]))
    y = cr.linear_fwd(bf16_to_dev(x), qw, sw, None if bias is None else bf16_to_dev(bias),
                      out=gy.t, workspace=gws.t)
    gy.check("y")
    gws.check("workspace")
    oqw, osw, _ = orc.rotate_quantize(w)
    ref = orc.linear_fwd(x, oqw, osw, bias=bias, rows=rows)
    yb = bits(y)
    if rows is not None:
        yb = yb[rows]
    return yb, ref


def test_linear_fwd_tiny(cr, orc):
    t = wl.tiny(0)
    say("linear_fwd tiny")
    yb, ref = _fwd_case(cr, orc, t["x"], t["w"])
    assert_rows_close(yb, ref["y"], "y")
    bias = wl.normal_bf16((t["N"],), 0.5, 0, 9)
    yb, ref = _fwd_case(cr, orc, t["x"], t["w"], bias=bias)
    assert_rows_close(yb, ref["y"], "y+bias")
    # elementwise: one fp32 product chain + bf16 rounding vs one rounding in fp64
    g = wl.bf16_bits_to_f32(yb).astype(np.float64)
    r = wl.bf16_bits_to_f32(ref["y"]).astype(np.float64)
    assert np.all(np.abs(g - r) <= 2.0 ** -7 * np.abs(r) + 1e-30)


# the longest contraction the row quantizer takes (CONVROT_MAX_ROW_LEN = 32768):
# the few-row path (5 rows), the small tiles (300 rows) and the 256 x 256 tiles
# with a ragged N (2100 rows)
@pytest.mark.parametrize("M,N,K", [(5, 384, 32768), (300, 640, 32768), (2100, 700, 32768)])
def test_linear_fwd_max_row_length(cr, orc, M, N, K):
    say(f"linear_fwd max row length M={M} N={N} K={K}")
    x = wl.activations(M, K, wl.n_outliers(K), base=M + 1)
    w = wl.normal_bf16((N, K), wl.SIGMA_W, M + 1, 1)
    yb, ref = _fwd_case(cr, orc, x, w)
    assert_rows_close(yb, ref["y"], "y")
    assert_fwd_elementwise(yb, ref["y"], "y")


@pytest.mark.parametrize("M,N,K", [(64, 32768, 256), (40, 256, 32768)])
def test_bwd_max_row_length(cr, orc, M, N, K):
    # dY rows of the longest length the dY quantizer takes (N = 32768, 16 waves
    # per row), and an input gradient 32768 wide (the inverse rotation over 256
    # blocks per row)
    say(f"bwd max row length M={M} N={N} K={K}")
    dy = wl.normal_bf16((M, N), wl.SIGMA_DY, N, 3)
    w = wl.normal_bf16((N, K), wl.SIGMA_W, N, 1)
    _bwd_int8(cr, orc, dy, w)
    _bwd_bf16(cr, orc, dy, w)


def test_many_rows(cr, orc):
    """A million-odd token rows of a short contraction: the row quantizers' and
    GEMMs' grids at their largest in this suite (over a million rows, tens of
    thousands of workgroups), checked on seeded sampled rows and both ends."""
    M, K, N = (1 << 20) + 3, 256, 136
    say(f"many rows M={M} K={K} N={N}")
    x = wl.activations(M, K, 3, base=77)
    w = wl.normal_bf16((N, K), wl.SIGMA_W, 77, 1)
    qw, sw = cr.quantize_weight(bf16_to_dev(w))
    xd = bf16_to_dev(x)
    qx, sx = cr.quantize_act(xd)
    y = cr.linear_fwd(xd, qw, sw)
    rows = np.unique(np.concatenate([[0, 1, M - 2, M - 1],
                                     np.random.default_rng(77).choice(M, 500, False)]))
    oqw, osw, _ = orc.rotate_quantize(w)
    oqx, osx, _ = orc.rotate_quantize(x[rows])
    rows_t = torch.from_numpy(rows).cuda()
    assert_exact(host(qx[rows_t]), oqx, "q_x (sampled rows)")
    assert_exact(host(sx[rows_t]), osx, "s_x (sampled rows)")
    oy = orc.dequant_epilogue(orc.gemm_i8_i32(oqx, oqw), osx, osw)
    assert_rows_close(bits(y[rows_t]), oy, "y (sampled rows)")
    assert_fwd_elementwise(bits(y[rows_t]), oy, "y (sampled rows)")
    # both input gradients through dY rows of 128 values (N = 128)
    w2 = wl.normal_bf16((128, K), wl.SIGMA_W, 78, 1)
    dy = wl.normal_bf16((M, 128), wl.SIGMA_DY, 78, 3)
    qw2, sw2 = cr.quantize_weight(bf16_to_dev(w2))
    oqw2, osw2, _ = orc.rotate_quantize(w2)
    dyd = bf16_to_dev(dy)
    for mode, ref in ((cr.BWD_INT8, orc.bwd_dx_int8), (cr.BWD_BF16, orc.bwd_dx_bf16)):
        dx = cr.linear_bwd_dx(dyd, qw2, sw2, mode)
        assert_rows_close(bits(dx[rows_t]), ref(dy[rows], oqw2, osw2)["dx"], f"dX mode {mode}")
    del xd, dyd


@pytest.mark.parametrize("M,N,K", [(1, 8, 128), (5, 130, 256), (300, 260, 384), (257, 1000, 1024)])
def test_linear_fwd_ragged(cr, orc, M, N, K):
    say(f"linear_fwd ragged M={M} N={N} K={K}")
    x = wl.activations(M, K, max(1, K // 100), base=M)
    w = wl.normal_bf16((N, K), wl.SIGMA_W, M, 1)
    yb, ref = _fwd_case(cr, orc, x, w)
    assert_rows_close(yb, ref["y"], "y")
    assert_fwd_elementwise(yb, ref["y"], "y")


def test_linear_fwd_attn_full_size(cr, orc):
    """The attention-projection workload at full size, the configuration the
    headline measures: all codes, scales and int32 accumulators exact, every
    output within the row tolerance and one bf16 ulp elementwise."""
    a = wl.attn(0)
    say("linear_fwd attn 4096^3")
    xd, wd = bf16_to_dev(a["x"]), bf16_to_dev(a["w"])
    qw, sw = cr.quantize_weight(wd)
    qx, sx = cr.quantize_act(xd)
    y = cr.linear_fwd(xd, qw, sw)
    y2 = cr.linear_fwd(xd, qw, sw)
    torch.cuda.synchronize()
    assert torch.equal(y, y2), "forward not deterministic"
    oqw, osw, bad = orc.rotate_quantize(a["w"])
    assert bad == 0
    assert_exact(host(qw), oqw, "q_w")
    assert_exact(host(sw), osw, "s_w")
    oqx, osx, bad = orc.rotate_quantize(a["x"])
    assert bad == 0
    assert_exact(host(qx), oqx, "q_x")
    assert_exact(host(sx), osx, "s_x")
    acc = cr.gemm_i8_i32(qx, qw, 0)
    oacc = orc.gemm_i8_i32(oqx, oqw)
    assert_exact(host(acc), oacc, "acc (all rows)")
    oy = orc.dequant_epilogue(oacc, osx, osw)
    e = assert_rows_close(bits(y), oy, "y (all rows)")
    assert_fwd_elementwise(bits(y), oy, "y (all rows)")
    say(f"  max row relerr {e:.2e}")


# --------------------------------------------------------------------------
# Input gradients
# --------------------------------------------------------------------------

@pytest.mark.parametrize("M,N", [(33, 256), (17, 1152), (9, 2048), (7, 4224), (5, 16384),
                                 (3, 24576), (3, 24704), (2, 32768)])
def test_bwd_quant_dy_exact(cr, orc, M, N):
    # the dY quantizer on both row plans: short rows packed into a span with the
    # column scales staged beside it, and rows of 2048 values or more folded one
    # row per workgroup (1, 2, 3, 8, 12, 13 and 16 waves)
    say(f"bwd_quant_dy M={M} N={N}")
    dy = wl.normal_bf16((M, N), 1e-3, 11, N % 1000)
    sw = (np.random.default_rng(N).random(N) * 1e-3 + 1e-5).astype(np.float32)
    qg, sg = cr.bwd_quant_dy(bf16_to_dev(dy), torch.from_numpy(sw).cuda())
    oqg, osg = orc.bwd_quant_dy(dy, sw)
    assert_exact(host(sg), osg, "s_g")
    assert_exact(host(qg), oqg, "q_g")


@pytest.mark.parametrize("N", [256, 1152, 2048, 4224, 32768])
def test_bwd_quant_dy_crafted_rows(cr, orc, N):
    # the quantizer's corner rows (all zero, exact ties, IEEE-division scales)
    # through the fold; power-of-two column scales keep the folded ties exact
    say(f"bwd_quant_dy crafted rows N={N}")
    dy = crafted_rows(N)
    sw = np.ldexp(np.ones(N, np.float32), -(np.arange(N) % 7)).astype(np.float32)
    qg, sg = cr.bwd_quant_dy(bf16_to_dev(dy), torch.from_numpy(sw).cuda())
    oqg, osg = orc.bwd_quant_dy(dy, sw)
    assert osg[0] == 0 and not oqg[0].any()
    assert_exact(host(sg), osg, "s_g")
    assert_exact(host(qg), oqg, "q_g")


@pytest.mark.parametrize("N", [256, 1152, 2048, 4096, 16384])
def test_bwd_quant_dy_subnormal_scales(cr, orc, N):
    # folded row maxima across fp32's subnormal binades: scales subnormal or zero,
    # the maximum's quotient past 127.5 (clamped to 127), and (N = 4096) column
    # scales that round the fold itself onto the subnormal grid
    say(f"bwd_quant_dy subnormal scales N={N}")
    dy, sw = tiny_fold_rows(N, N)
    if N == 4096:
        sw = (np.random.default_rng(2).uniform(0.5, 1.0, N) * 2.0 ** -20).astype(np.float32)
    gq, gs = Guarded(dy.shape, torch.int8), Guarded((dy.shape[0],), torch.float32)
    qg, sg = cr.bwd_quant_dy(bf16_to_dev(dy), torch.from_numpy(sw).cuda(), out=(gq.t, gs.t))
    gq.check("q_g")
    gs.check("s_g")
    oqg, osg = orc.bwd_quant_dy(dy, sw)
    assert (osg == 0).any() and ((osg > 0) & (osg < 2.0 ** -126)).any()
    assert_exact(host(sg), osg, "s_g")
    assert_exact(host(qg), oqg, "q_g")


def _bwd_int8(cr, orc, dy, w, rows=None):
    qw, sw = cr.quantize_weight(bf16_to_dev(w))
    oqw, osw, _ = orc.rotate_quantize(w)
    dyd = bf16_to_dev(dy)
    qg, sg = cr.bwd_quant_dy(dyd, sw)
    M, N, K = dy.shape[0], dy.shape[1], w.shape[1]
    gdx = Guarded((M, K), torch.bfloat16)
    gws = guarded_workspace(cr.workspace_bytes(cr.OP_LINEAR_BWD_DX, M, N, K, cr.BWD_INT8))
    dx = cr.linear_bwd_dx(dyd, qw, sw, cr.BWD_INT8, out=gdx.t, workspace=gws.t)
    gdx.check("dX int8")
    gws.check("workspace (int8 dX)")
    oqg, osg = orc.bwd_quant_dy(dy, osw)
    assert_exact(host(sg), osg, "s_g")
    assert_exact(host(qg), oqg, "q_g")
    acc2 = cr.gemm_i8_i32(qg, qw, 1)
    oacc2 = orc.gemm_i8_i32_rows_of_b(oqg, oqw, rows)
    g = host(acc2) if rows is None else host(acc2)[rows]
    assert_exact(g, oacc2, "acc2")
    odx = orc.bwd_int8_epilogue(oacc2, osg, rows)
    dxb = bits(dx) if rows is None else bits(dx)[rows]
    return assert_rows_close(dxb, odx, "dX int8")


def _bwd_bf16(cr, orc, dy, w, rows=None):
    qw, sw = cr.quantize_weight(bf16_to_dev(w))
    oqw, osw, _ = orc.rotate_quantize(w)
    gwt = Guarded((w.shape[1], w.shape[0]), torch.bfloat16)
    wt = cr.dequant_weight_t(qw, sw, out=gwt.t)
    gwt.check("W_hat^T")
    owhat = orc.dequant_weight(oqw, osw)
    assert_rows_close(bits(wt), np.ascontiguousarray(owhat.T), "W_hat^T")
    M, N, K = dy.shape[0], dy.shape[1], w.shape[1]
    gdx = Guarded((M, K), torch.bfloat16)
    gws = guarded_workspace(cr.workspace_bytes(cr.OP_LINEAR_BWD_DX, M, N, K, cr.BWD_BF16))
    dx = cr.linear_bwd_dx(bf16_to_dev(dy), qw, sw, cr.BWD_BF16, out=gdx.t, workspace=gws.t)
    gdx.check("dX bf16")
    gws.check("workspace (bf16 dX)")
    odx = orc.bf16_gemm_dx(dy, owhat, rows)
    dxb = bits(dx) if rows is None else bits(dx)[rows]
    return assert_rows_close(dxb, odx, "dX bf16")


def test_bwd_int8_tiny(cr, orc):
    t = wl.tiny(0)
    say("bwd int8 tiny")
    _bwd_int8(cr, orc, t["dy"], t["w"])


def test_bwd_bf16_tiny(cr, orc):
    t = wl.tiny(0)
    say("bwd bf16 tiny")
    _bwd_bf16(cr, orc, t["dy"], t["w"])


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (300, 384, 640), (257, 1024, 512)])
def test_bwd_ragged(cr, orc, M, N, K):
    say(f"bwd ragged M={M} N={N} K={K}")
    dy = wl.normal_bf16((M, N), wl.SIGMA_DY, M, 3)
    dy[0] = 0  # an all-zero gradient row
    w = wl.normal_bf16((N, K), wl.SIGMA_W, M, 1)
    _bwd_int8(cr, orc, dy, w)
    _bwd_bf16(cr, orc, dy, w)


# --------------------------------------------------------------------------
# Embedding
# --------------------------------------------------------------------------

@pytest.mark.parametrize("V,D,T", [(1000, 4096, 300), (77, 384, 50), (10, 128, 7), (300, 8192, 40),
                                   (200, 4224, 33), (500, 1152, 5003)])
def test_embedding_lookup(cr, orc, V, D, T):
    say(f"embedding V={V} D={D} T={T}")
    E = wl.normal_bf16((V, D), wl.SIGMA_W, V, 1)
    qe, se = cr.quantize_weight(bf16_to_dev(E), chunk_rows=64)
    oqe, ose, _ = orc.rotate_quantize(E, chunk_rows=64)
    assert_exact(host(qe), oqe, "q_E")
    assert_exact(host(se), ose, "s_E")
    ids = wl.token_ids(T, V, base=D)
    ids[0], ids[-1] = -5, V   # out of range -> zero rows, counted
    oob = torch.zeros(1, dtype=torch.int32, device="cuda")
    gout = Guarded((T, D), torch.bfloat16)
    out = cr.embedding_lookup(to_dev(ids), qe, se, oob, out=gout.t)
    gout.check("lookup")
    oout, ooob = orc.embedding_lookup(ids, oqe, ose)
    assert int(oob.item()) == ooob == 2
    ob = bits(out)
    assert not ob[0].any() and not ob[-1].any()
    assert_rows_close(ob, oout, "lookup")


def test_embedding_lookup_many_ids(cr, orc):
    # 300000 ids: each persistent lookup wave handles ~73 tokens, so every wave
    # fetches its next 64 ids again mid-stream; out-of-range ids are spread
    # through the stream, among repeated ones
    V, D, T = 1000, 128, 300000
    say(f"embedding lookup V={V} D={D} T={T}")
    E = wl.normal_bf16((V, D), wl.SIGMA_W, 11, 1)
    qe, se = cr.quantize_weight(bf16_to_dev(E))
    oqe, ose, _ = orc.rotate_quantize(E)
    ids = wl.token_ids(T, V, base=11)
    g = np.random.default_rng(11)
    bad = g.choice(T, 500, replace=False)
    ids[bad] = np.where(g.random(500) < 0.5, -1 - g.integers(0, 1 << 20, 500), V + g.integers(0, 1 << 20, 500))
    oob = torch.zeros(1, dtype=torch.int32, device="cuda")
    gout = Guarded((T, D), torch.bfloat16)
    out = cr.embedding_lookup(to_dev(ids), qe, se, oob, out=gout.t)
    gout.check("lookup")
    oout, ooob = orc.embedding_lookup(ids, oqe, ose)
    assert int(oob.item()) == ooob == 500
    ob = bits(out)
    assert not ob[bad].any()
    assert_rows_close(ob, oout, "lookup")


def test_binding_rejects_mismatched_buffers(cr):
    """The binding checks every tensor against the sizes it passes to the C ABI
    (which sees only pointers) and raises before anything is enqueued."""
    d = "cuda"
    x = torch.zeros((64, 256), dtype=torch.bfloat16, device=d)
    qw = torch.zeros((128, 256), dtype=torch.int8, device=d)
    sw = torch.ones((128,), dtype=torch.float32, device=d)
    bad = [
        lambda: cr.linear_fwd(x, qw, sw[:64]),                                   # scales too short
        lambda: cr.linear_fwd(x, qw[:, :128].contiguous(), sw),                  # K mismatch
        lambda: cr.linear_fwd(x, qw, sw, bias=torch.zeros(64, dtype=torch.bfloat16, device=d)),
        lambda: cr.linear_fwd(x, qw, sw, out=torch.empty((64, 64), dtype=torch.bfloat16, device=d)),
        lambda: cr.linear_fwd(x, qw, sw, workspace=torch.empty(16, dtype=torch.uint8, device=d)),
        lambda: cr.quantize_weight(x, out=(torch.empty((64, 128), dtype=torch.int8, device=d),
                                           torch.empty((64,), dtype=torch.float32, device=d))),
        lambda: cr.gemm_i8_i32(qw, qw[:64].contiguous(), 0),                    # fine shapes ...
    ]
    for i, fn in enumerate(bad[:-1]):
        with pytest.raises(ValueError):
            fn()
    torch.cuda.synchronize()
    # ... and a well-formed call still works afterwards
    acc = bad[-1]()
    torch.cuda.synchronize()
    assert tuple(acc.shape) == (128, 64) and int(acc.abs().max().item()) == 0


def test_empty_batch(cr):
    """A batch of 0 tokens / rows / ids goes through every entry point as a no-op
    and returns empty outputs of the right shape; the lookup leaves its
    out-of-range counter alone."""
    say("empty batch through every entry point")
    d = "cuda"
    K, N = 4096, 512
    w = bf16_to_dev(wl.packed_weight(77, 0, N, K))
    qw, sw = cr.quantize_weight(w)
    x0 = torch.empty((0, K), dtype=torch.bfloat16, device=d)
    dy0 = torch.empty((0, N), dtype=torch.bfloat16, device=d)
    a = torch.zeros((16, K), dtype=torch.bfloat16, device=d)
    b = torch.zeros((N, 16), dtype=torch.bfloat16, device=d)
    q0, s0 = cr.quantize_weight(x0)
    assert tuple(q0.shape) == (0, K) and tuple(s0.shape) == (0,)
    qa, sa = cr.quantize_act(x0)
    assert tuple(qa.shape) == (0, K) and tuple(sa.shape) == (0,)
    assert tuple(cr.linear_fwd(x0, qw, sw).shape) == (0, N)
    assert tuple(cr.linear_fwd_lora(x0, qw, sw, a, b, 0.5).shape) == (0, N)
    assert tuple(cr.lora_down(x0, a).shape) == (0, 16)
    assert tuple(cr.gemm_i8_bf16(qa, sa, qw, sw).shape) == (0, N)
    assert tuple(cr.gemm_i8_i32(qa, qw).shape) == (0, N)
    qg, sg = cr.bwd_quant_dy(dy0, sw)
    assert tuple(qg.shape) == (0, N) and tuple(sg.shape) == (0,)
    for mode in (cr.BWD_BF16, cr.BWD_INT8):
        assert tuple(cr.linear_bwd_dx(dy0, qw, sw, mode).shape) == (0, K)
    oob = torch.full((1,), 7, dtype=torch.int32, device=d)
    out = cr.embedding_lookup(torch.empty((0,), dtype=torch.int32, device=d), qw, sw, oob)
    torch.cuda.synchronize()
    assert tuple(out.shape) == (0, K) and int(oob.item()) == 7
    # the layer still works after the empty calls
    x = bf16_to_dev(wl.activations(3, K, wl.n_outliers(K), base=1))
    assert torch.equal(cr.linear_fwd(x, qw, sw), cr.gemm_i8_bf16(*cr.quantize_act(x), qw, sw))
