"""LoRA branch of the forward ("LoRA Training Guide for MOSS-Image", section 7.1,
ConvRot INT8 scope bullet: the quantized layers stay LoRA-trainable and the
LoRA branch receives the unrotated input).

Compared with the oracle (O13):
  * xa = bf16(x . A^T): rows within the 1e-2 row tolerance (the GPU accumulates
    in fp32, the oracle in binary64, so a bf16 rounding may land one ulp apart);
  * y: int32 accumulators bit-exact (same GEMM as the plain forward), outputs
    within the 1e-2 row tolerance of the oracle's LoRA epilogue;
  * a zero up projection or a zero scale gives the plain forward bit for bit.
Shapes: the tiny layer (64 x 256 x 256), ragged ones (301 x 384 x 640; one row
at K = 128, where most down-projection waves have no k-block; 7 x 8192 x 1000,
two load groups per wave; 259 x 4224 x 300), both ranks 16 and 32, and sampled
rows of the attention projection (4096^3, rank 16).
"""
import numpy as np
import pytest

import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from gpu_util import assert_exact, assert_rows_close, bf16_to_dev, bits, host  # noqa: E402


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


def _case(M, K, N, R, base):
    x = wl.activations(M, K, wl.n_outliers(K), base=base)
    w = wl.packed_weight(3000 + R, base, N, K)
    lw = wl.lora_weights(K, N, R, base)
    return x, w, lw["a"], lw["b"]


@pytest.mark.parametrize("M,K,N", [(64, 256, 256), (301, 384, 640), (1, 128, 100),
                                   (7, 8192, 1000), (259, 4224, 300)])
@pytest.mark.parametrize("R", [16, 32])
def test_lora_small(cr, orc, M, K, N, R):
    x, w, a, b = _case(M, K, N, R, 0)
    scale = 0.75
    qw, sw = cr.quantize_weight(bf16_to_dev(w))
    xd, ad, bd = bf16_to_dev(x), bf16_to_dev(a), bf16_to_dev(b)
    xa = cr.lora_down(xd, ad)
    oxa = orc.lora_down(x, a)
    assert_rows_close(bits(xa), oxa, "xa")
    y = cr.linear_fwd_lora(xd, qw, sw, ad, bd, scale)
    oqx, osx, _ = orc.rotate_quantize(x)
    oqw, osw, _ = orc.rotate_quantize(w)
    qx, _ = cr.quantize_act(xd)
    assert_exact(host(cr.gemm_i8_i32(qx, qw, 0)), orc.gemm_i8_i32(oqx, oqw), "acc")
    ref = orc.lora_epilogue(orc.gemm_i8_i32(oqx, oqw), osx, osw, oxa, b, scale)
    e = assert_rows_close(bits(y), ref, "y")
    print(f"  max row relerr {e:.2e}", flush=True)


def test_lora_zero_branch_is_plain_forward(cr):
    x, w, a, b = _case(64, 256, 256, 16, 1)
    qw, sw = cr.quantize_weight(bf16_to_dev(w))
    xd, ad = bf16_to_dev(x), bf16_to_dev(a)
    y0 = cr.linear_fwd(xd, qw, sw)
    zero_b = torch.zeros((256, 16), dtype=torch.bfloat16, device="cuda")
    assert torch.equal(cr.linear_fwd_lora(xd, qw, sw, ad, zero_b, 1.0), y0)
    assert torch.equal(cr.linear_fwd_lora(xd, qw, sw, ad, bf16_to_dev(b), 0.0), y0)


def test_lora_with_bias(cr, orc):
    x, w, a, b = _case(64, 256, 256, 32, 2)
    bias = wl.normal_bf16((256,), 1.0, 2, 17)
    qw, sw = cr.quantize_weight(bf16_to_dev(w))
    xd = bf16_to_dev(x)
    y = cr.linear_fwd_lora(xd, qw, sw, bf16_to_dev(a), bf16_to_dev(b), 0.5, bias=bf16_to_dev(bias))
    oqx, osx, _ = orc.rotate_quantize(x)
    oqw, osw, _ = orc.rotate_quantize(w)
    ref = orc.lora_epilogue(orc.gemm_i8_i32(oqx, oqw), osx, osw, orc.lora_down(x, a), b, 0.5,
                            bias=bias)
    assert_rows_close(bits(y), ref, "y (bias)")


def test_lora_attention_projection(cr, orc):
    at = wl.attn(0)
    x, w = at["x"], at["w"]
    lw = wl.lora_weights(4096, 4096, 16, 0)
    a, b = lw["a"], lw["b"]
    qw, sw = cr.quantize_weight(bf16_to_dev(w))
    xd = bf16_to_dev(x)
    y = cr.linear_fwd_lora(xd, qw, sw, bf16_to_dev(a), bf16_to_dev(b), 1.0)
    g = np.random.default_rng(61)
    rows = np.unique(np.concatenate([[0, 4095], g.choice(4096, 14, replace=False)]))
    oqx, osx, _ = orc.rotate_quantize(x)
    oqw, osw, _ = orc.rotate_quantize(w)
    oxa = orc.lora_down(x, a, rows)
    xa = cr.lora_down(xd, bf16_to_dev(a))
    assert_rows_close(bits(xa)[rows], oxa, "xa (sampled rows)")
    ref = orc.lora_epilogue(orc.gemm_i8_i32(oqx, oqw, rows), osx, osw, oxa, b, 1.0, rows=rows)
    e = assert_rows_close(bits(y)[rows], ref, "y (sampled rows)")
    print(f"  max row relerr {e:.2e}", flush=True)
