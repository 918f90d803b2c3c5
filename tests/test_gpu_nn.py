"""The PyTorch modules (w8a8_rotated_int8_amd.nn) against the C-ABI calls they wrap.

ConvRotLinear and ConvRotEmbedding only reshape and check arguments, so their
outputs and input gradients must equal the direct calls bit for bit; the direct
calls are compared with the oracle in the other GPU tests, and the tiny forward
is compared with the oracle here as well.
"""
import numpy as np
import pytest

import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from gpu_util import assert_rows_close, bf16_to_dev, bits  # noqa: E402


@pytest.fixture(scope="module")
def cr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import w8a8_rotated_int8_amd as cr
    cr.lib()
    return cr


def same(a, b, what):
    assert a.shape == b.shape, (what, a.shape, b.shape)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)), what


@pytest.mark.parametrize("bias", [False, True])
@pytest.mark.parametrize("mode", ["bf16", "int8"])
def test_linear_module_forward_backward(cr, bias, mode):
    from w8a8_rotated_int8_amd.nn import ConvRotLinear
    N, K = 640, 384
    print(f"ConvRotLinear N={N} K={K} bias={bias} mode={mode}", flush=True)
    lin = torch.nn.Linear(K, N, bias=bias, dtype=torch.bfloat16, device="cuda")
    with torch.no_grad():
        lin.weight.copy_(bf16_to_dev(wl.packed_weight(71, 0, N, K)))
        if bias:
            lin.bias.copy_(bf16_to_dev(wl.activations(1, N, 0, base=72)[0]))
    mod = ConvRotLinear.from_linear(lin, bwd_mode=mode)
    qw, sw = cr.quantize_weight(lin.weight.detach())
    assert torch.equal(mod.qw, qw) and torch.equal(mod.sw, sw)
    assert not any(p.requires_grad for p in mod.parameters())

    x = bf16_to_dev(wl.activations(2 * 37, K, wl.n_outliers(K), base=73)).reshape(2, 37, K)
    x.requires_grad_(True)
    y = mod(x)
    assert y.shape == (2, 37, N) and y.dtype == torch.bfloat16
    b = lin.bias.detach() if bias else None
    same(y.detach().reshape(-1, N), cr.linear_fwd(x.detach().reshape(-1, K), qw, sw, b), "forward")

    gy = bf16_to_dev(wl.activations(2 * 37, N, 0, base=74)).reshape(2, 37, N)
    (gx,) = torch.autograd.grad(y, x, gy)
    ref = cr.linear_bwd_dx(gy.reshape(-1, N), qw, sw, cr.BWD_BF16 if mode == "bf16" else cr.BWD_INT8)
    same(gx.reshape(-1, K), ref, "input gradient")


def test_linear_module_matches_oracle(cr):
    import oracle
    from w8a8_rotated_int8_amd.nn import ConvRotLinear
    t = wl.tiny(0)
    mod = ConvRotLinear(*cr.quantize_weight(bf16_to_dev(t["w"])))
    y = mod(bf16_to_dev(t["x"]))
    oqw, osw, _ = oracle.rotate_quantize(t["w"])
    assert_rows_close(bits(y), oracle.linear_fwd(t["x"], oqw, osw)["y"], "module forward")


def test_linear_module_with_lora_branch(cr):
    """A LoRA branch wrapped around the frozen layer sees the unrotated input and
    receives gradients; the base contributes grad_x only."""
    from w8a8_rotated_int8_amd.nn import ConvRotLinear
    N, K, R = 256, 256, 16
    t = wl.tiny(1)
    mod = ConvRotLinear(*cr.quantize_weight(bf16_to_dev(t["w"])))
    a = torch.nn.Parameter(0.01 * torch.randn(R, K, device="cuda", dtype=torch.bfloat16))
    bb = torch.nn.Parameter(0.01 * torch.randn(N, R, device="cuda", dtype=torch.bfloat16))
    x = bf16_to_dev(t["x"]).requires_grad_(True)
    y = mod(x) + (x @ a.t()) @ bb.t()
    y.float().square().sum().backward()
    assert a.grad is not None and bb.grad is not None and x.grad is not None
    assert torch.isfinite(a.grad.float()).all() and torch.isfinite(x.grad.float()).all()


def test_linear_module_empty_batch(cr):
    from w8a8_rotated_int8_amd.nn import ConvRotLinear
    t = wl.tiny(0)
    mod = ConvRotLinear(*cr.quantize_weight(bf16_to_dev(t["w"])))
    x = torch.zeros((0, 256), dtype=torch.bfloat16, device="cuda", requires_grad=True)
    y = mod(x)
    assert y.shape == (0, 256)
    (gx,) = torch.autograd.grad(y, x, torch.zeros_like(y))
    assert gx.shape == (0, 256)


def test_embedding_module(cr):
    from w8a8_rotated_int8_amd.nn import ConvRotEmbedding
    V, D = 700, 512
    print(f"ConvRotEmbedding V={V} D={D}", flush=True)
    emb = torch.nn.Embedding(V, D, dtype=torch.bfloat16, device="cuda")
    with torch.no_grad():
        emb.weight.copy_(bf16_to_dev(wl.packed_weight(81, 0, V, D)))
    mod = ConvRotEmbedding.from_embedding(emb, chunk_rows=128)
    qe, se = cr.quantize_weight(emb.weight.detach())
    assert torch.equal(mod.qe, qe) and torch.equal(mod.se, se), "chunked != unchunked"

    ids = torch.from_numpy(wl.token_ids(3 * 11, V, base=82).astype(np.int64)).view(3, 11).cuda()
    ids[0, 4] = -5
    ids[2, 7] = V
    ids[1, 1] = 2**33 + 3  # would wrap to 3 if narrowed without a range check
    out = mod(ids)
    assert out.shape == (3, 11, D)
    i32 = ids.reshape(-1).clamp(-1, V).to(torch.int32)
    ref = cr.embedding_lookup(i32, qe, se)
    same(out.reshape(-1, D), ref, "lookup")
    for r, c in ((0, 4), (2, 7), (1, 1)):
        assert not out[r, c].float().abs().any(), (r, c)

    strict = ConvRotEmbedding(qe, se, check_ids=True)
    with pytest.raises(IndexError):
        strict(ids)
    ok = ids.clone()
    ok[0, 4], ok[2, 7], ok[1, 1] = 1, 2, 3
    same(strict(ok.to(torch.int32)), mod(ok), "int32 and int64 ids")
