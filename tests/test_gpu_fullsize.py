"""GPU parity at the full workload sizes, through the same C-ABI calls bench.py
times.  Quantizers are compared in full (bit-exact codes and scales).  The int8
GEMMs of the MLP pair and of the first packed layer are compared on every row
(bit-exact int32 accumulators, outputs within the 1e-2 row tolerance and the
forward's one-ulp elementwise bound); the other packed layers and the bf16
input gradients on seeded sampled rows that the oracle computes one by one.
The oracle's accumulators of the input gradient, sum_n q_g[m][n] q_w[n][k],
come from its row-major triple loop applied to q_w transposed (the same sums,
in the same order over n).

Workloads: the MLP pair (up [16384,4096], down [4096,16384], 4096 tokens; the
down input is the bf16 GELU of the unquantized up projection), the packed
20480-token stream (layers 0, 251 and two seeded others of the 252), and the
248320-row token embedding quantized in 8192-row chunks with a 32768-id lookup.
"""
import numpy as np
import pytest

import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from gpu_util import (assert_exact, assert_fwd_elementwise, assert_rows_close, bf16_to_dev,  # noqa: E402
                      bits, host, to_dev)


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


def say(*a):
    print(*a, flush=True)


def sample_rows(M, n, seed):
    g = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, M - 1], g.choice(M, n, replace=False)]))


# --------------------------------------------------------------------------
# MLP pair
# --------------------------------------------------------------------------

@pytest.fixture(scope="module")
def mlp(cr, orc):
    say("mlp: generating x, W_up, W_down (numpy recipe)")
    x = wl.activations(4096, 4096, wl.n_outliers(4096), base=0)
    w = wl.mlp_weights(0)

    def gpu_matmul(a, b):
        return (torch.from_numpy(a).cuda() @ torch.from_numpy(b).cuda().T).cpu().numpy()

    h = wl.mlp_down_input(x, w["w_up"], matmul=gpu_matmul)
    g = wl.mlp_grads(4096, 0)
    say("mlp: oracle weight quantization")
    oq_up, os_up, b1 = orc.rotate_quantize(w["w_up"])
    oq_dn, os_dn, b2 = orc.rotate_quantize(w["w_down"])
    assert b1 == 0 and b2 == 0
    return dict(x=x, h=h, w_up=w["w_up"], w_down=w["w_down"], dy_down=g["dy_down"],
                dy_up=g["dy_up"], oq_up=oq_up, os_up=os_up, oq_dn=oq_dn, os_dn=os_dn)


def test_mlp_weight_quantization_exact(cr, mlp):
    say("mlp: weight quantization parity")
    for name, oq, os_ in (("w_up", "oq_up", "os_up"), ("w_down", "oq_dn", "os_dn")):
        q, s = cr.quantize_weight(bf16_to_dev(mlp[name]))
        assert_exact(host(s), mlp[os_], f"{name} scales")
        assert_exact(host(q), mlp[oq], f"{name} codes")


@pytest.mark.parametrize("which", ["up", "down"])
def test_mlp_forward(cr, orc, mlp, which):
    xin = mlp["x"] if which == "up" else mlp["h"]
    wkey = "w_up" if which == "up" else "w_down"
    oq, os_ = (mlp["oq_up"], mlp["os_up"]) if which == "up" else (mlp["oq_dn"], mlp["os_dn"])
    say(f"mlp {which}: forward M=4096 K={xin.shape[1]} N={oq.shape[0]}")
    qw, sw = cr.quantize_weight(bf16_to_dev(mlp[wkey]))
    xd = bf16_to_dev(xin)
    y = cr.linear_fwd(xd, qw, sw)
    qx, sx = cr.quantize_act(xd)
    oqx, osx, bad = orc.rotate_quantize(xin)
    if which == "up":
        assert bad == 0
    else:
        # GELU of strongly negative pre-activations leaves values down to ~1e-30
        # beside values ~10 in the same block: the binary64 sums round (the
        # oracle's witness counts every row), so the exact-sum reading does not
        # hold and the summation order could in principle move a last bit of r.
        # Codes and scales are still compared bit for bit.
        say(f"  rows with inexact binary64 rotation sums: {bad} of {xin.shape[0]}")
    assert_exact(host(sx), osx, "s_x")
    assert_exact(host(qx), oqx, "q_x")
    acc = cr.gemm_i8_i32(qx, qw, 0)
    say("  oracle int32 GEMM, every row")
    oacc = orc.gemm_i8_i32(oqx, oq)
    assert_exact(host(acc), oacc, "acc (all rows)")
    oy = orc.dequant_epilogue(oacc, osx, os_)
    e = assert_rows_close(bits(y), oy, "y (all rows)")
    assert_fwd_elementwise(bits(y), oy, "y (all rows)")
    say(f"  max row relerr {e:.2e}")


@pytest.mark.parametrize("which", ["down", "up"])
def test_mlp_int8_grad(cr, orc, mlp, which):
    # down layer: dY [4096,4096] -> dX [4096,16384]; up layer: dY [4096,16384] -> dX [4096,4096]
    dy = mlp["dy_down"] if which == "down" else mlp["dy_up"]
    wkey = "w_down" if which == "down" else "w_up"
    oq, os_ = (mlp["oq_dn"], mlp["os_dn"]) if which == "down" else (mlp["oq_up"], mlp["os_up"])
    say(f"mlp {which}: int8 dX N={dy.shape[1]} K={oq.shape[1]}")
    qw, sw = cr.quantize_weight(bf16_to_dev(mlp[wkey]))
    dyd = bf16_to_dev(dy)
    dx = cr.linear_bwd_dx(dyd, qw, sw, cr.BWD_INT8)
    qg, sg = cr.bwd_quant_dy(dyd, sw)
    oqg, osg = orc.bwd_quant_dy(dy, os_)
    assert_exact(host(sg), osg, "s_g")
    assert_exact(host(qg), oqg, "q_g")
    acc2 = cr.gemm_i8_i32(qg, qw, 1)
    say("  oracle int32 GEMM along q_w's rows, every row")
    oacc2 = orc.gemm_i8_i32(oqg, np.ascontiguousarray(oq.T))
    assert_exact(host(acc2), oacc2, "acc2 (all rows)")
    e = assert_rows_close(bits(dx), orc.bwd_int8_epilogue(oacc2, osg), "dX int8 (all rows)")
    say(f"  max row relerr {e:.2e}")


@pytest.mark.parametrize("which", ["down", "up"])
def test_mlp_bf16_grad(cr, orc, mlp, which):
    dy = mlp["dy_down"] if which == "down" else mlp["dy_up"]
    wkey = "w_down" if which == "down" else "w_up"
    oq, os_ = (mlp["oq_dn"], mlp["os_dn"]) if which == "down" else (mlp["oq_up"], mlp["os_up"])
    say(f"mlp {which}: bf16 dX")
    qw, sw = cr.quantize_weight(bf16_to_dev(mlp[wkey]))
    dx = cr.linear_bwd_dx(bf16_to_dev(dy), qw, sw, cr.BWD_BF16)
    owhat = orc.dequant_weight(oq, os_)
    wt = cr.dequant_weight_t(qw, sw)
    cols = sample_rows(owhat.shape[0], 60, 31)          # rows of W_hat = columns of W_hat^T
    assert_rows_close(np.ascontiguousarray(bits(wt).T[cols]), owhat[cols], "W_hat (sampled rows)")
    rows = sample_rows(4096, 6, 32 if which == "down" else 33)
    e = assert_rows_close(bits(dx)[rows], orc.bf16_gemm_dx(dy, owhat, rows), "dX bf16")
    say(f"  max row relerr {e:.2e}")


# --------------------------------------------------------------------------
# Packed 20480-token stream
# --------------------------------------------------------------------------

@pytest.fixture(scope="module")
def packed(orc):
    say("packed: generating x [20480,4096] and dY")
    p = wl.packed(0)
    oqx, osx, bad = orc.rotate_quantize(p["x"])
    assert bad == 0
    return dict(p=p, oqx=oqx, osx=osx)


def test_packed_activation_quantization(cr, packed):
    say("packed: q_x of 20480 rows")
    qx, sx = cr.quantize_act(bf16_to_dev(packed["p"]["x"]))
    assert_exact(host(sx), packed["osx"], "s_x")
    assert_exact(host(qx), packed["oqx"], "q_x")


@pytest.mark.parametrize("layer", [0, 251, 97, 180])
def test_packed_layer(cr, orc, packed, layer):
    p = packed["p"]
    say(f"packed: layer {layer} forward + int8 and bf16 dX on 20480 tokens")
    w = wl.packed_weight(layer, 0)
    oq, os_, _ = orc.rotate_quantize(w)
    qw, sw = cr.quantize_weight(bf16_to_dev(w))
    assert_exact(host(sw), os_, "s_w")
    assert_exact(host(qw), oq, "q_w")
    xd = bf16_to_dev(p["x"])
    y = cr.linear_fwd(xd, qw, sw)
    qx, _ = cr.quantize_act(xd)
    # the first layer on every row, the others on seeded sampled rows
    rows = np.arange(20480) if layer == 0 else sample_rows(20480, 22, 40 + layer)
    acc = cr.gemm_i8_i32(qx, qw, 0)
    oacc = orc.gemm_i8_i32(packed["oqx"], oq, None if layer == 0 else rows)
    assert_exact(host(acc)[rows], oacc, "acc")
    oy = orc.dequant_epilogue(oacc, packed["osx"], os_, None if layer == 0 else rows)
    assert_rows_close(bits(y)[rows], oy, "y")
    assert_fwd_elementwise(bits(y)[rows], oy, "y")
    dyd = bf16_to_dev(p["dy"])
    dx = cr.linear_bwd_dx(dyd, qw, sw, cr.BWD_INT8)
    qg, sg = cr.bwd_quant_dy(dyd, sw)
    oqg, osg = orc.bwd_quant_dy(p["dy"], os_)
    assert_exact(host(sg), osg, "s_g")
    assert_exact(host(qg), oqg, "q_g")
    acc2 = cr.gemm_i8_i32(qg, qw, 1)
    if layer == 0:
        oacc2 = orc.gemm_i8_i32(oqg, np.ascontiguousarray(oq.T))
        assert_exact(host(acc2), oacc2, "acc2 (all rows)")
        assert_rows_close(bits(dx), orc.bwd_int8_epilogue(oacc2, osg), "dX int8 (all rows)")
    else:
        oacc2 = orc.gemm_i8_i32_rows_of_b(oqg, oq, rows)
        assert_exact(host(acc2)[rows], oacc2, "acc2")
        assert_rows_close(bits(dx)[rows], orc.bwd_int8_epilogue(oacc2, osg, rows), "dX int8")
    # the default backward: transient bf16 W_hat, bf16 GEMM over the 20480 tokens
    dx16 = cr.linear_bwd_dx(dyd, qw, sw, cr.BWD_BF16)
    owhat = orc.dequant_weight(oq, os_)
    e = assert_rows_close(bits(dx16)[rows], orc.bf16_gemm_dx(p["dy"], owhat, rows), "dX bf16")
    say(f"  bf16 dX max row relerr {e:.2e}")


# --------------------------------------------------------------------------
# Token embedding 248320 x 4096
# --------------------------------------------------------------------------

@pytest.mark.timeout(900)
def test_embedding_full(cr, orc):
    V, D, CH, T = wl.EMBED_V, wl.EMBED_D, wl.EMBED_CHUNK, wl.EMBED_T
    say(f"embedding: generating E [{V},{D}] (numpy recipe)")
    E = wl.embed_table(0)
    Ed = bf16_to_dev(E)
    q, s = cr.quantize_weight(Ed, chunk_rows=CH)
    q1, s1 = cr.quantize_weight(Ed)                    # unchunked: identical
    assert torch.equal(q, q1) and torch.equal(s, s1)
    del q1, s1
    g = np.random.default_rng(7)
    edges = np.array([0, 1, CH - 1, CH, CH + 1, 2 * CH - 1, 30 * CH - 1, 30 * CH, V - 2, V - 1])
    rows = np.unique(np.concatenate([edges, g.choice(V, 4000, replace=False)]))
    say(f"embedding: oracle on {rows.size} sampled rows")
    oq, os_, bad = orc.rotate_quantize(E[rows])
    assert bad == 0
    rows_t = torch.from_numpy(rows).cuda()
    assert_exact(host(s[rows_t]), os_, "s_E (sampled rows)")
    assert_exact(host(q[rows_t]), oq, "q_E (sampled rows)")
    say(f"embedding: lookup of {T} ids")
    ids = wl.embed_ids(0)
    oob = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = cr.embedding_lookup(to_dev(ids), q, s, oob)
    assert int(oob.item()) == 0
    tok = np.unique(np.concatenate([[0, T - 1], g.choice(T, 600, replace=False)]))
    sel = ids[tok]
    oq2, os2, _ = orc.rotate_quantize(E[sel])
    ref, n_oob = orc.embedding_lookup(np.arange(sel.size, dtype=np.int32), oq2, os2)
    assert n_oob == 0
    e = assert_rows_close(bits(out)[tok], ref, "lookup (sampled tokens)")
    say(f"  max row relerr {e:.2e}")
