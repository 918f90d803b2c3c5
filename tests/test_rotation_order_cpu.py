"""The kernels' butterfly order against the oracle's index-order sums, on rows
where binary64 sums are not exact.

The rotation r_j = fl32(fl64(S_j * c)), S_j = sum_i H[i][j] x_i, is independent
of the order of the additions whenever every partial sum is exact in binary64.
The MLP down input (the bf16 GELU of the up projection, exact erf) breaks that:
GELU of strongly negative pre-activations leaves values near 1e-30 beside values
near 10 in one block, and the oracle's exactness witness counts every row.

The kernels evaluate S by a fast Walsh-Hadamard transform: the butterfly
stages pair element bits 0, 1, 2, 3, 4 inside a lane, then bit 5 and bit 6
across lanes, each stage forming a + b and a - b in binary64 (a the partner
with the bit clear).  This test runs exactly that sequence of binary64
operations in numpy on the whole MLP down input of the seeded recipe
(4096 x 16384).  Where a binary64 partial sum rounds, the two orders may round
differently, so r itself can differ in its last fp32 bit: on this input 2 of
the 67,108,864 values do, by one ulp.  The test pins what the layer's parity
bar needs: codes and scales equal to the oracle's on every row, and any
difference in r at most one ulp on at most a handful of values.

Source: "LoRA Training Guide for MOSS-Image", section 7.1, "ConvRot INT8"
(block-diagonal Hadamard rotation of the activations, row-wise int8
quantization); the block size 128 and the normalisation are this layer's
readings.
"""
import numpy as np
import pytest

import workloads as wl

C128 = float.fromhex("0x1.6a09e667f3bcdp-4")


def butterfly_rotate(x_bits: np.ndarray) -> np.ndarray:
    """fl32(fl64(S * c)) with S from the kernels' butterfly order (stage h = 1,
    2, 4, ..., 64 of the 128-point transform), in binary64."""
    M, K = x_bits.shape
    v = wl.bf16_bits_to_f32(x_bits).astype(np.float64).reshape(M, K // 128, 128)
    h = 1
    while h < 128:
        w = v.reshape(M, K // 128, 128 // (2 * h), 2, h)
        a = w[:, :, :, 0, :]
        b = w[:, :, :, 1, :]
        v = np.stack([a + b, a - b], axis=3).reshape(M, K // 128, 128)
        h *= 2
    return (v * C128).astype(np.float32).reshape(M, K)


def test_butterfly_matches_index_order_when_sums_are_exact(oracle_mod):
    x = wl.activations(64, 4096, wl.n_outliers(4096), base=3)
    r, bad = oracle_mod.rotate_rows(x)
    assert bad == 0
    assert np.array_equal(butterfly_rotate(x).view(np.uint32), r.view(np.uint32))


def test_butterfly_order_pinned_by_unit_vectors():
    # e1 rotates to alternating +-c (natural Sylvester order), e64 to 64 x (+c)
    # then 64 x (-c): a wrong stage pairing or sign would move them.
    c = np.float32(C128)
    for i, expect in ((1, np.tile([c, -c], 64)), (64, np.repeat([c, -c], 64))):
        e = np.zeros((1, 128), np.float32)
        e[0, i] = 1.0
        got = butterfly_rotate(wl.f32_to_bf16_bits(e))[0]
        assert np.array_equal(got, expect.astype(np.float32))


@pytest.mark.slow
def test_mlp_down_input_rotation_is_order_independent(oracle_mod):
    x = wl.activations(4096, 4096, wl.n_outliers(4096), base=0)
    w_up = wl.mlp_weights(0)["w_up"]
    h = wl.mlp_down_input(x, w_up)
    del x, w_up
    M, K = h.shape
    inexact_total = 0
    r_diffs = 0
    step = 256
    for r0 in range(0, M, step):
        hb = h[r0:r0 + step]
        r_ref, bad = oracle_mod.rotate_rows(hb)
        inexact_total += bad
        r_bfly = butterfly_rotate(hb)
        d = r_bfly.view(np.uint32) != r_ref.view(np.uint32)
        if d.any():
            ulps = np.abs(r_bfly.view(np.int32)[d].astype(np.int64) - r_ref.view(np.int32)[d])
            assert ulps.max() == 1, (r0, ulps.max())
            r_diffs += int(d.sum())
        q_ref, s_ref = oracle_mod.quantize_rows(r_ref)
        q_b, s_b = oracle_mod.quantize_rows(r_bfly)
        assert np.array_equal(q_ref, q_b) and np.array_equal(s_ref.view(np.uint32),
                                                              s_b.view(np.uint32))
    # the rows really are outside the exact-sum reading, and the orders do differ
    assert inexact_total == M
    assert r_diffs <= 16, r_diffs
