"""Shared-input projections: q, k and v weights stacked into one [3N, K] code
matrix are served by one activation quantization and one GEMM ("LoRA Training
Guide for MOSS-Image", the transformer block's proj.q/k/v linears, which read
the same normalized input; per-row scales make the stacking exact).

On the attention-projection input (x [4096, 4096], 41 outlier columns x50) with
three seeded [4096, 4096] weights:
  * the stacked call's output column blocks equal the three separate calls'
    outputs bit for bit;
  * the stacked weight codes and scales equal the oracle's, and sampled output
    rows match the oracle (bit-exact int32 accumulators, 1e-2 row tolerance).
"""
import numpy as np
import pytest

import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from gpu_util import (assert_exact, assert_fwd_elementwise, assert_rows_close, bf16_to_dev,  # noqa: E402
                      bits, host)


@pytest.fixture(scope="module")
def cr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import w8a8_rotated_int8_amd as cr
    cr.lib()
    return cr


@pytest.fixture(scope="module")
def qkv(cr):
    print("qkv: generating x [4096,4096] and three [4096,4096] weights", flush=True)
    a = wl.attn(0)
    ws = wl.qkv_weights(0)
    N, K = ws[0].shape
    qcat = torch.empty((3 * N, K), dtype=torch.int8, device="cuda")
    scat = torch.empty((3 * N,), dtype=torch.float32, device="cuda")
    for j, w in enumerate(ws):   # load-time quantization straight into the stacked buffer
        cr.quantize_weight(bf16_to_dev(w), out=(qcat[j * N:(j + 1) * N], scat[j * N:(j + 1) * N]))
    return dict(x=a["x"], ws=ws, N=N, K=K, qcat=qcat, scat=scat)


def test_stacked_equals_separate(cr, qkv):
    N = qkv["N"]
    xd = bf16_to_dev(qkv["x"])
    y = cr.linear_fwd(xd, qkv["qcat"], qkv["scat"])
    assert tuple(y.shape) == (xd.shape[0], 3 * N)
    for j, w in enumerate(qkv["ws"]):
        qw, sw = cr.quantize_weight(bf16_to_dev(w))
        assert torch.equal(qw, qkv["qcat"][j * N:(j + 1) * N])
        assert torch.equal(sw, qkv["scat"][j * N:(j + 1) * N])
        yj = cr.linear_fwd(xd, qw, sw)
        assert torch.equal(y[:, j * N:(j + 1) * N], yj), f"projection {j}"


def test_stacked_vs_oracle(cr, qkv):
    import oracle
    N = qkv["N"]
    wcat = np.concatenate(qkv["ws"], axis=0)
    oq, os_, bad = oracle.rotate_quantize(wcat)
    assert bad == 0
    assert_exact(host(qkv["scat"]), os_, "stacked s_w")
    assert_exact(host(qkv["qcat"]), oq, "stacked q_w")
    oqx, osx, bad = oracle.rotate_quantize(qkv["x"])
    assert bad == 0
    xd = bf16_to_dev(qkv["x"])
    y = cr.linear_fwd(xd, qkv["qcat"], qkv["scat"])
    qx, _ = cr.quantize_act(xd)
    g = np.random.default_rng(51)
    rows = np.unique(np.concatenate([[0, 4095], g.choice(4096, 12, replace=False)]))
    acc = cr.gemm_i8_i32(qx, qkv["qcat"], 0)
    oacc = oracle.gemm_i8_i32(oqx, oq, rows)
    assert_exact(host(acc)[rows], oacc, "stacked acc (sampled rows)")
    oy = oracle.dequant_epilogue(oacc, osx, os_, rows)
    e = assert_rows_close(bits(y)[rows], oy, "stacked y")
    assert_fwd_elementwise(bits(y)[rows], oy, "stacked y")
    print(f"  max row relerr {e:.2e}", flush=True)
