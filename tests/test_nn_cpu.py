"""Host logic of the PyTorch modules (w8a8_rotated_int8_amd.nn), on the CPU.

The library calls are replaced by stand-ins that record their arguments and
return tensors of the right shape, so these tests check only what the modules
themselves do: reshaping to 2-D and back, contiguity, the backward mode passed
down, that the frozen buffers get no gradient, and the id handling of the
embedding.  The calls' numerics are the GPU tests' concern.
"""
import pytest

torch = pytest.importorskip("torch")

import w8a8_rotated_int8_amd.nn as crn  # noqa: E402


@pytest.fixture
def spy(monkeypatch):
    calls = []

    def fwd(x2, qw, sw, bias):
        calls.append(("fwd", tuple(x2.shape), x2.is_contiguous(), bias is not None))
        # row r holds the value r (exact in bf16)
        return torch.arange(x2.shape[0], dtype=torch.float32)[:, None].expand(
            x2.shape[0], qw.shape[0]).to(torch.bfloat16).contiguous()

    def bwd(gy, qw, sw, mode):
        calls.append(("bwd", tuple(gy.shape), gy.is_contiguous(), mode))
        return torch.full((gy.shape[0], qw.shape[1]), 2.0, dtype=torch.bfloat16)

    def lookup(ids, qe, se, oob):
        calls.append(("lookup", ids.dtype, tuple(ids.shape), ids.tolist(), oob is not None))
        return torch.zeros((ids.shape[0], qe.shape[1]), dtype=torch.bfloat16)

    monkeypatch.setattr(crn, "linear_fwd", fwd)
    monkeypatch.setattr(crn, "linear_bwd_dx", bwd)
    monkeypatch.setattr(crn, "embedding_lookup", lookup)
    return calls


@pytest.mark.parametrize("mode,code", [("bf16", 0), ("int8", 1)])
def test_linear_reshapes_and_routes_the_backward(spy, mode, code):
    N, K = 96, 256
    mod = crn.ConvRotLinear(torch.zeros((N, K), dtype=torch.int8), torch.ones(N),
                            torch.zeros(N, dtype=torch.bfloat16), bwd_mode=mode)
    base = torch.zeros((K, 3, 2), dtype=torch.bfloat16)
    x = base.permute(2, 1, 0).requires_grad_(True)  # [2, 3, K], not contiguous
    x.retain_grad()
    y = mod(x)
    assert y.shape == (2, 3, N)
    assert spy[0] == ("fwd", (6, K), True, True)
    # row r of the 2-D output is row r of the flattened leading dims
    assert bool((y[1, 1].float() == 4).all()) and bool((y[0, 2].float() == 2).all())
    y.float().sum().backward()
    assert spy[1] == ("bwd", (6, N), True, code)
    assert x.grad.shape == (2, 3, K) and bool((x.grad == 2).all())
    assert all(b.grad is None for b in mod.buffers())


def test_linear_without_input_grad_skips_the_backward(spy):
    mod = crn.ConvRotLinear(torch.zeros((128, 128), dtype=torch.int8), torch.ones(128))
    with torch.no_grad():
        mod(torch.zeros((5, 128), dtype=torch.bfloat16))
    mod(torch.zeros((5, 128), dtype=torch.bfloat16))
    assert [c[0] for c in spy] == ["fwd", "fwd"]


def test_embedding_ids(spy):
    V, D = 50, 128
    emb = crn.ConvRotEmbedding(torch.zeros((V, D), dtype=torch.int8), torch.ones(V))
    ids = torch.tensor([[0, 49, 50], [-7, 2**40, 3]], dtype=torch.int64)
    out = emb(ids)
    assert out.shape == (2, 3, D)
    kind, dt, shape, vals, counted = spy[-1]
    assert dt == torch.int32 and shape == (6,) and not counted
    # in-range ids unchanged; every bad id stays outside [0, V) after narrowing
    assert vals[:2] == [0, 49] and vals[5] == 3
    assert all(v < 0 or v >= V for v in (vals[2], vals[3], vals[4]))
    emb32 = crn.ConvRotEmbedding(torch.zeros((V, D), dtype=torch.int8), torch.ones(V), check_ids=True)
    emb32(torch.tensor([1, 2], dtype=torch.int32))
    assert spy[-1][1] == torch.int32 and spy[-1][4]
