"""Pins of the CPU oracle against what the mathematics and the pages fix.

The pages print no numeric worked example, so the oracle is pinned by closed
forms derived by hand below (each with its derivation), invariants of the
method, textbook/library special cases and brute force on tiny inputs.  Each
pin is chosen so that a plausible mistake (a dropped term, a wrong sign or
index, a transposed operand, a different Hadamard ordering, half-away rounding,
reciprocal instead of division) fails at least one of them.
"""
import math

import numpy as np
import pytest
import scipy.linalg

import workloads as wl

C128 = float.fromhex("0x1.6a09e667f3bcdp-4")     # 1/sqrt(128) as fl64(sqrt 2) * 2^-4
FL32_C = float.fromhex("0x1.6a09e6p-4")           # fl32 of it (derived: the 24th bit is 0, rest < half)


def hexeq(v, hexstr):
    return float(v) == float.fromhex(hexstr)


def bf16(vals):
    return wl.f32_to_bf16_bits(np.asarray(vals, dtype=np.float32))


def block_row(entries, K=128):
    v = np.zeros(K, dtype=np.float32)
    for i, val in entries.items():
        v[i] = val
    return bf16(v)[None, :]


# --------------------------------------------------------------------------
# P1: Hadamard matrix, normalisation constant
# --------------------------------------------------------------------------

@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 32, 64, 128])
def test_p1_sylvester_matches_closed_form_and_scipy(oracle_mod, n):
    H = oracle_mod.hadamard(n).astype(np.int64)
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    pop = np.vectorize(lambda v: bin(int(v)).count("1"))(i & j)
    assert np.array_equal(H, (-1) ** pop)                       # closed form (natural order)
    assert np.array_equal(H, scipy.linalg.hadamard(n))          # library Sylvester construction
    assert np.array_equal(H, H.T)
    assert np.array_equal(H @ H.T, n * np.eye(n, dtype=np.int64))


def test_p1_norm_constant(oracle_mod):
    c = oracle_mod.norm_const(128)
    assert c.hex() == "0x1.6a09e667f3bcdp-4"
    assert c == math.ldexp(math.sqrt(2.0), -4)
    assert c != 1.0 / math.sqrt(128.0)          # the double-rounded form is one ulp low
    assert abs(c * c * 128 - 1.0) < 4e-16
    assert oracle_mod.norm_const(1) == 1.0 and oracle_mod.norm_const(4) == 0.5
    H = oracle_mod.hadamard(128).astype(np.float64)
    R = H * c
    assert np.max(np.abs(R @ R.T - np.eye(128))) < 1e-15


# --------------------------------------------------------------------------
# P2: rotation identity x W^T = (xR)(WR)^T; rotation equals the library form
# --------------------------------------------------------------------------

def test_p2_rotation_preserves_inner_products(oracle_mod):
    t = wl.tiny(0)
    x, w = t["x"], t["w"]
    rx, bx = oracle_mod.rotate_rows(x)
    rw, bw = oracle_mod.rotate_rows(w)
    assert bx == 0 and bw == 0
    xf = wl.bf16_bits_to_f32(x).astype(np.float64)
    wf = wl.bf16_bits_to_f32(w).astype(np.float64)
    exact = xf @ wf.T
    rot = rx.astype(np.float64) @ rw.astype(np.float64).T
    # each rotated value carries one fp32 rounding (rel 2^-24) on top of an
    # exact fp64 sum and one fp64 rounding; bound the inner product error
    bound = 3 * 2.0 ** -24 * (np.abs(rx).astype(np.float64) @ np.abs(rw).astype(np.float64).T)
    assert np.all(np.abs(rot - exact) <= bound + 1e-12)
    # norms are preserved too (R orthogonal)
    assert np.allclose(np.linalg.norm(rx.astype(np.float64), axis=1),
                       np.linalg.norm(xf, axis=1), rtol=1e-6)


def test_p2_rotation_equals_library_matmul_when_exact(oracle_mod):
    x = wl.activations(16, 512, 8, base=3)
    r, bad = oracle_mod.rotate_rows(x)
    assert bad == 0
    xf = wl.bf16_bits_to_f32(x).astype(np.float64)
    H = scipy.linalg.hadamard(128).astype(np.float64)
    ref = np.concatenate([xf[:, b:b + 128] @ H for b in range(0, 512, 128)], axis=1)
    ref32 = (ref * C128).astype(np.float32)
    assert np.array_equal(r.view(np.uint32), ref32.view(np.uint32))


def test_p2_exactness_witness_trips_on_huge_spread(oracle_mod):
    row = block_row({0: 2.0 ** 60, 1: 2.0 ** -60, 5: 1.0})
    ok = block_row({0: 3.0, 1: -0.5})
    _, bad = oracle_mod.rotate_rows(np.concatenate([row, ok]))
    assert bad == 1


# --------------------------------------------------------------------------
# P3: quantizer bounds
# --------------------------------------------------------------------------

def test_p3_quantizer_bounds(oracle_mod):
    x = wl.activations(64, 1024, 10, base=5)
    r, _ = oracle_mod.rotate_rows(x)
    q, s = oracle_mod.quantize_rows(r)
    assert q.min() >= -127 and q.max() <= 127
    am = np.argmax(np.abs(r), axis=1)
    assert np.all(np.abs(q[np.arange(64), am]) == 127)
    err = np.abs(r.astype(np.float64) - q.astype(np.float64) * s[:, None].astype(np.float64))
    assert np.all(err <= (s[:, None].astype(np.float64) / 2) * (1 + 2.0 ** -22))
    assert np.all(s == (np.max(np.abs(r), axis=1) / np.float32(127)).astype(np.float32))


def test_p3_zero_row(oracle_mod):
    x = np.zeros((3, 256), dtype=np.uint16)
    x[1, 7] = bf16([1.5])[0]
    q, s, _ = oracle_mod.rotate_quantize(x)
    assert s[0] == 0 and s[2] == 0 and not q[0].any() and not q[2].any()
    assert s[1] > 0


# --------------------------------------------------------------------------
# P4: symmetry, equivariance, row independence, chunking
# --------------------------------------------------------------------------

def test_p4_sign_and_power_of_two_equivariance(oracle_mod):
    x = wl.activations(32, 512, 5, base=7)
    q, s, _ = oracle_mod.rotate_quantize(x)
    qn, sn, _ = oracle_mod.rotate_quantize(x ^ np.uint16(0x8000))
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)
    for k in (-3, 1, 4):
        xs = bf16(wl.bf16_bits_to_f32(x) * np.float32(2.0 ** k))   # exact: power-of-two scale
        qk, sk, _ = oracle_mod.rotate_quantize(xs)
        assert np.array_equal(qk, q)
        assert np.array_equal(sk, (s * np.float32(2.0 ** k)).astype(np.float32))


def test_p4_rows_are_independent_and_chunking_is_invisible(oracle_mod):
    x = wl.activations(50, 384, 4, base=9)
    q, s, _ = oracle_mod.rotate_quantize(x)
    perm = np.random.default_rng(1).permutation(50)
    qp, sp, _ = oracle_mod.rotate_quantize(x[perm])
    assert np.array_equal(qp, q[perm]) and np.array_equal(sp, s[perm])
    qs, ss, _ = oracle_mod.rotate_quantize(x[10:27])          # row slice (qkv split)
    assert np.array_equal(qs, q[10:27]) and np.array_equal(ss, s[10:27])
    for chunk in (1, 7, 16, 49, 50, 64):
        qc, sc, _ = oracle_mod.rotate_quantize(x, chunk_rows=chunk)
        assert np.array_equal(qc, q) and np.array_equal(sc, s)


# --------------------------------------------------------------------------
# P5: block 1 reduces ConvRot to plain symmetric per-row int8
# --------------------------------------------------------------------------

def test_p5_block1_is_plain_rowwise_int8(oracle_mod):
    # worked example: a = 254, s = 2, t = [127, 0.5, -1.5, 63.5] -> half-even
    x = bf16([[254.0, 1.0, -3.0, 127.0]])
    q, s, _ = oracle_mod.rotate_quantize(x, block=1)
    assert s[0] == 2.0
    assert q.tolist() == [[127, 0, -2, 64]]                  # half-away would give 1 for 0.5
    # library special case on random rows: numpy fp32 division + rint (half-even)
    xr = wl.activations(40, 96, 3, base=11)
    q, s, _ = oracle_mod.rotate_quantize(xr, block=1)
    xf = wl.bf16_bits_to_f32(xr)
    sref = (np.max(np.abs(xf), axis=1) / np.float32(127)).astype(np.float32)
    qref = np.clip(np.rint(xf / sref[:, None]), -127, 127).astype(np.int8)
    assert np.array_equal(s, sref) and np.array_equal(q, qref)


# --------------------------------------------------------------------------
# P6 - P9: block-128 closed forms (ordering, normalisation, ties, division)
# --------------------------------------------------------------------------

def test_p6_unit_vectors_fix_order_and_normalisation(oracle_mod):
    # e0: every column of H has H[0][j] = 1 -> all r_j = fl32(c), all codes 127
    q, s, _ = oracle_mod.rotate_quantize(block_row({0: 1.0}))
    assert np.all(q == 127) and hexeq(s[0], "0x1.6ce3aep-11")
    r, _ = oracle_mod.rotate_rows(block_row({0: 1.0}))
    assert np.all(r == np.float32(FL32_C))
    # ones: only column 0 sums to 128, the others cancel -> r_0 = fl32(128 c)
    q, s, _ = oracle_mod.rotate_quantize(block_row({i: 1.0 for i in range(128)}))
    assert q[0, 0] == 127 and not q[0, 1:].any() and hexeq(s[0], "0x1.6ce3aep-4")
    # e1: H[1][j] = (-1)^j -> alternating (natural order; sequency order differs)
    q, _, _ = oracle_mod.rotate_quantize(block_row({1: 1.0}))
    assert q[0].tolist() == [127, -127] * 64
    # e64: H[64][j] = (-1)^[j >= 64]
    q, _, _ = oracle_mod.rotate_quantize(block_row({64: 1.0}))
    assert q[0].tolist() == [127] * 64 + [-127] * 64
    # a second block is rotated independently of the first
    x = np.concatenate([block_row({1: 1.0}), block_row({64: -2.0})], axis=1)
    q, _, _ = oracle_mod.rotate_quantize(x)
    assert q[0, :128].tolist() == [64, -64] * 64 and q[0, 128:].tolist() == [-127] * 64 + [127] * 64


def test_p7_tie_rounds_half_to_even(oracle_mod):
    # x = -253 e0 - 255 e1: S_even = -508, S_odd = 2; 508 = 4*127 so
    # s = 4 fl32(c) and t_odd = 2 fl32(c) / s = 0.5 exactly -> RNE gives 0
    q, s, _ = oracle_mod.rotate_quantize(block_row({0: -253.0, 1: -255.0}))
    assert hexeq(s[0], "0x1.6a09e6p-2")
    assert q[0].tolist() == [-127, 0] * 64


def test_p8_tie_at_63_5(oracle_mod):
    # x = 3 e0 + e1: S_even = 4, S_odd = 2 -> t_odd = 63.5 exactly -> 64
    q, s, _ = oracle_mod.rotate_quantize(block_row({0: 3.0, 1: 1.0}))
    assert hexeq(s[0], "0x1.6ce3aep-9")
    assert q[0].tolist() == [127, 64] * 64


def test_p9_division_not_reciprocal(oracle_mod):
    # x = -255 e0 - 85 e1: S = -340 / -170; t_odd = fl32(r/s) = -63.5 -> -64,
    # whereas r * fl32(127/a) = -63.499996 would give -63
    q, s, _ = oracle_mod.rotate_quantize(block_row({0: -255.0, 1: -85.0}))
    assert hexeq(s[0], "0x1.e49e62p-3")
    assert q[0].tolist() == [-127, -64] * 64


# --------------------------------------------------------------------------
# P10: int32 GEMM
# --------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (3, 5, 256), (8, 8, 256), (7, 2, 1)])
def test_p10_int_gemm_matches_numpy(oracle_mod, M, N, K):
    g = np.random.default_rng(M * 100 + N)
    a = g.integers(-127, 128, (M, K), dtype=np.int8)
    b = g.integers(-127, 128, (N, K), dtype=np.int8)
    acc = oracle_mod.gemm_i8_i32(a, b)
    assert np.array_equal(acc, a.astype(np.int64) @ b.astype(np.int64).T)
    rows = [M - 1, 0]
    assert np.array_equal(oracle_mod.gemm_i8_i32(a, b, rows), acc[rows])


def test_p10_gemm_extreme_magnitude(oracle_mod):
    K = 16384
    a = np.full((2, K), -127, dtype=np.int8)
    b = np.full((3, K), -127, dtype=np.int8)
    b[1] = 127
    acc = oracle_mod.gemm_i8_i32(a, b)
    assert acc[0, 0] == 127 * 127 * K and acc[0, 1] == -127 * 127 * K
    assert abs(int(acc.max())) < 2 ** 31


def test_rows_of_b_gemm_is_transpose_contraction(oracle_mod):
    g = np.random.default_rng(5)
    qg = g.integers(-127, 128, (6, 40), dtype=np.int8)
    qw = g.integers(-127, 128, (40, 256), dtype=np.int8)
    acc2 = oracle_mod.gemm_i8_i32_rows_of_b(qg, qw)
    assert np.array_equal(acc2, qg.astype(np.int64) @ qw.astype(np.int64))
    assert np.array_equal(oracle_mod.gemm_i8_i32_rows_of_b(qg, qw, [4]), acc2[[4]])


# --------------------------------------------------------------------------
# Rounding helpers
# --------------------------------------------------------------------------

def test_rne_integer(oracle_mod):
    for t, e in [(0.5, 0), (1.5, 2), (2.5, 2), (-0.5, 0), (-1.5, -2), (-2.5, -2), (63.5, 64),
                 (64.5, 64), (126.5, 126), (0.49999997, 0), (-127.0, -127), (3.7, 4), (-3.7, -4)]:
        assert oracle_mod.rne_integer(t) == e
    vals = np.random.default_rng(0).uniform(-200, 200, 2000)
    assert all(oracle_mod.rne_integer(v) == np.rint(v) for v in vals)


def _bf16_neighbours(x):
    f = np.float32(x)
    u = int(np.array([f]).view(np.uint32)[0])
    lo = (u >> 16) & 0xFFFF
    return lo, (lo + 1) & 0xFFFF


def test_double_to_bf16_brute_force(oracle_mod):
    g = np.random.default_rng(2)
    xs = list(g.standard_normal(3000) * 10.0 ** g.integers(-8, 8, 3000))
    # exact ties: 1 + 2^-8 -> 1 (even), 1 + 3*2^-8 -> 1 + 2^-6 (even mantissa)
    assert oracle_mod.double_to_bf16(1.0 + 2.0 ** -8) == 0x3F80
    assert oracle_mod.double_to_bf16(1.0 + 3 * 2.0 ** -8) == 0x3F82
    assert oracle_mod.double_to_bf16(-(1.0 + 2.0 ** -8 + 2.0 ** -40)) == 0xBF81
    for x in xs:
        b = oracle_mod.double_to_bf16(x)
        v = float(wl.bf16_bits_to_f32(np.array([b], dtype=np.uint16))[0])
        cands = []
        for nb in _bf16_neighbours(x) + _bf16_neighbours(np.nextafter(np.float32(x), np.float32(0))):
            cands.append(float(wl.bf16_bits_to_f32(np.array([nb], dtype=np.uint16))[0]))
        best = min(abs(c - x) for c in cands)
        assert abs(v - x) == best
        if sum(abs(c - x) == best for c in set(cands)) > 1:
            assert b % 2 == 0


# --------------------------------------------------------------------------
# O8: dequantization epilogue
# --------------------------------------------------------------------------

def test_o8_epilogue_is_nearest_bf16_of_the_exact_product(oracle_mod):
    t = wl.tiny(0)
    qw, sw, _ = oracle_mod.rotate_quantize(t["w"])
    bias = bf16(np.linspace(-1, 1, t["N"]))
    out = oracle_mod.linear_fwd(t["x"], qw, sw, bias=bias)
    v = (out["acc"].astype(np.float64) * out["sx"][:, None].astype(np.float64)
         * sw[None, :].astype(np.float64) + wl.bf16_bits_to_f32(bias)[None, :].astype(np.float64))
    y = wl.bf16_bits_to_f32(out["y"]).astype(np.float64)
    assert np.all(np.abs(y - v) <= 2.0 ** -8 * np.abs(v) + 1e-30)
    # the quantized layer approximates the bf16 layer (the method's purpose)
    xf = wl.bf16_bits_to_f32(t["x"]).astype(np.float64)
    wf = wl.bf16_bits_to_f32(t["w"]).astype(np.float64)
    ref = xf @ wf.T + wl.bf16_bits_to_f32(bias)[None, :]
    rel = np.linalg.norm(y - ref, axis=1) / np.linalg.norm(ref, axis=1)
    assert np.max(rel) < 0.05


# --------------------------------------------------------------------------
# O9 / O10: the two input-gradient paths
# --------------------------------------------------------------------------

def _dequantized_unrotated_weight(oracle_mod, qw, sw):
    c = oracle_mod.norm_const(128)
    H = scipy.linalg.hadamard(128).astype(np.float64)
    wr = qw.astype(np.float64) * sw[:, None].astype(np.float64)
    K = qw.shape[1]
    return np.concatenate([wr[:, b:b + 128] @ H * c for b in range(0, K, 128)], axis=1)


def test_o9_int8_grad_is_dy_times_dequantized_weight(oracle_mod):
    t = wl.tiny(0)
    qw, sw, _ = oracle_mod.rotate_quantize(t["w"])
    res = oracle_mod.bwd_dx_int8(t["dy"], qw, sw)
    What = _dequantized_unrotated_weight(oracle_mod, qw, sw)
    dyf = wl.bf16_bits_to_f32(t["dy"]).astype(np.float64)
    ref = dyf @ What
    dx = wl.bf16_bits_to_f32(res["dx"]).astype(np.float64)
    # error budget: dY quantization (s_g/2 per element, through |q_w|) + bf16 output
    qerr = (res["sg"][:, None].astype(np.float64) / 2) * np.sqrt(
        (np.abs(qw.astype(np.float64)) ** 2).sum(axis=0))[None, :] * np.sqrt(t["N"])
    rowerr = np.linalg.norm(dx - ref, axis=1)
    assert np.all(rowerr <= np.linalg.norm(qerr, axis=1) + 2.0 ** -8 * np.linalg.norm(ref, axis=1))
    rel = rowerr / np.linalg.norm(ref, axis=1)
    assert np.max(rel) < 0.03
    # the intermediate quantities obey the quantizer's own bounds
    g = (wl.bf16_bits_to_f32(t["dy"]) * sw[None, :]).astype(np.float32)
    assert np.array_equal(res["sg"], (np.max(np.abs(g), axis=1) / np.float32(127)).astype(np.float32))
    assert np.array_equal(res["acc2"], res["qg"].astype(np.int64) @ qw.astype(np.int64))


def test_o10_bf16_grad_is_dy_times_dequantized_weight(oracle_mod):
    t = wl.tiny(0)
    qw, sw, _ = oracle_mod.rotate_quantize(t["w"])
    res = oracle_mod.bwd_dx_bf16(t["dy"], qw, sw)
    What = _dequantized_unrotated_weight(oracle_mod, qw, sw)
    wh = wl.bf16_bits_to_f32(res["what"]).astype(np.float64)
    assert np.all(np.abs(wh - What) <= 2.0 ** -8 * np.abs(What) + 1e-30)
    dyf = wl.bf16_bits_to_f32(t["dy"]).astype(np.float64)
    ref = dyf @ wh
    dx = wl.bf16_bits_to_f32(res["dx"]).astype(np.float64)
    assert np.all(np.abs(dx - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-30)
    # dequantized weight approximates the original bf16 weight (rotation undone)
    wf = wl.bf16_bits_to_f32(t["w"]).astype(np.float64)
    assert np.max(np.linalg.norm(wh - wf, axis=1) / np.linalg.norm(wf, axis=1)) < 0.05


# --------------------------------------------------------------------------
# P11: embedding round trip; O11 lookup
# --------------------------------------------------------------------------

def test_p11_embedding_round_trip(oracle_mod):
    V, D = 300, 512
    E = wl.normal_bf16((V, D), wl.SIGMA_W, 4, 1)
    qe, se, bad = oracle_mod.rotate_quantize(E, chunk_rows=64)
    assert bad == 0
    ids = np.array([0, 299, 17, 17, -1, 300, 5], dtype=np.int32)
    out, oob = oracle_mod.embedding_lookup(ids, qe, se)
    assert oob == 2 and not out[4].any() and not out[5].any()
    assert np.array_equal(out[2], out[3])
    Ef = wl.bf16_bits_to_f32(E).astype(np.float64)
    of = wl.bf16_bits_to_f32(out).astype(np.float64)
    for t, i in enumerate(ids):
        if 0 <= i < V:
            err = np.linalg.norm(of[t] - Ef[i])
            bound = (se[i] / 2) * math.sqrt(D) * (1 + 2.0 ** -20) + 2.0 ** -8 * np.linalg.norm(of[t])
            assert err <= bound
    # without the inverse rotation the rows would not match
    raw = qe[ids[0]].astype(np.float64) * se[ids[0]]
    assert np.linalg.norm(raw - Ef[ids[0]]) > 0.5 * np.linalg.norm(Ef[ids[0]])


# --------------------------------------------------------------------------
# P12: outlier smoothing (report + weak sanity bound)
# --------------------------------------------------------------------------

def test_p12_rotation_smooths_outliers(oracle_mod):
    x = wl.activations(64, 4096, wl.n_outliers(4096), base=0)
    xf = wl.bf16_bits_to_f32(x).astype(np.float64)
    q, s, _ = oracle_mod.rotate_quantize(x)
    c = oracle_mod.norm_const(128)
    H = scipy.linalg.hadamard(128).astype(np.float64)
    xhat_rot = q.astype(np.float64) * s[:, None]
    xhat = np.concatenate([xhat_rot[:, b:b + 128] @ H * c for b in range(0, 4096, 128)], axis=1)
    q1, s1, _ = oracle_mod.rotate_quantize(x, block=1)
    xhat1 = q1.astype(np.float64) * s1[:, None]
    e_rot = np.linalg.norm(xhat - xf)
    e_plain = np.linalg.norm(xhat1 - xf)
    print(f"rotated int8 error {e_rot:.3f} vs plain per-row int8 {e_plain:.3f}")
    assert e_rot < 0.5 * e_plain


def test_oracle_regression_digests(oracle_mod):
    import json
    import os
    import sys
    here = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
    sys.path.insert(0, here)
    import make_golden
    with open(os.path.join(here, "tiny_oracle_digests.json")) as f:
        stored = json.load(f)
    assert make_golden.digests() == stored


# --------------------------------------------------------------------------
# O13: LoRA branch (down projection to bf16, up projection in the epilogue)
# --------------------------------------------------------------------------

def _bf16(vals):
    return wl.f32_to_bf16_bits(np.asarray(vals, dtype=np.float32))


def test_lora_down_worked_example(oracle_mod):
    # x = [1, 2], A = [[3, 4], [-0.5, 0.25]]: xa = [1*3 + 2*4, -0.5 + 0.5] = [11, 0]
    x = _bf16([[1.0, 2.0]])
    a = _bf16([[3.0, 4.0], [-0.5, 0.25]])
    xa = oracle_mod.lora_down(x, a)
    assert xa.tolist() == _bf16([[11.0, 0.0]]).tolist()


def test_lora_down_rounds_once_to_bf16(oracle_mod):
    # bf16 spacing above 1 is 2^-7: 1 + 2^-8 is the midpoint (tie -> even, 1.0),
    # 1 + 3*2^-9 lies above it (-> 1 + 2^-7); both sums are exact in binary64
    x = _bf16([[1.0, 1.0]])
    a = _bf16([[1.0, 2.0 ** -8], [1.0, 3 * 2.0 ** -9]])
    xa = oracle_mod.lora_down(x, a)
    assert xa[0].tolist() == _bf16([1.0, 1.0 + 2.0 ** -7]).tolist()


def test_lora_down_one_hot_is_identity(oracle_mod):
    g = np.random.default_rng(3)
    K, R = 256, 16
    x = _bf16(g.standard_normal((5, K)))
    a = np.zeros((R, K), dtype=np.uint16)
    a[np.arange(R), 7 * np.arange(R)] = _bf16([1.0])[0]
    xa = oracle_mod.lora_down(x, a)
    assert np.array_equal(xa, x[:, 7 * np.arange(R)])
    # rows subset
    xa2 = oracle_mod.lora_down(x, a, rows=[4, 1])
    assert np.array_equal(xa2, xa[[4, 1]])


def test_lora_epilogue_zero_branch_is_base(oracle_mod):
    g = np.random.default_rng(4)
    acc = g.integers(-30000, 30000, (3, 8), dtype=np.int32)
    sx = (g.random(3) + 0.1).astype(np.float32) * 1e-3
    sw = (g.random(8) + 0.1).astype(np.float32) * 1e-3
    bias = _bf16(g.standard_normal(8))
    xa = _bf16(g.standard_normal((3, 16)))
    base = oracle_mod.dequant_epilogue(acc, sx, sw, bias=bias)
    zero_b = np.zeros((8, 16), dtype=np.uint16)
    assert np.array_equal(oracle_mod.lora_epilogue(acc, sx, sw, xa, zero_b, 0.75, bias=bias), base)
    b = _bf16(g.standard_normal((8, 16)))
    assert np.array_equal(oracle_mod.lora_epilogue(acc, sx, sw, xa, b, 0.0, bias=bias), base)


def test_lora_epilogue_worked_example(oracle_mod):
    # acc = 0: y = bf16(scale * sum_r xa_r * B_nr); xa = [2, -1], B = [[0.5, 1], [3, 0]]
    acc = np.zeros((1, 2), dtype=np.int32)
    sx = np.ones(1, dtype=np.float32)
    sw = np.ones(2, dtype=np.float32)
    xa = _bf16([[2.0, -1.0]])
    b = _bf16([[0.5, 1.0], [3.0, 0.0]])
    y = oracle_mod.lora_epilogue(acc, sx, sw, xa, b, 0.25)
    assert y.tolist() == _bf16([[0.0, 1.5]]).tolist()
    # with a base term: acc 100 * 0.5 * 0.25 = 12.5, plus 0.25 * [0, 6]
    acc2 = np.full((1, 2), 100, dtype=np.int32)
    y2 = oracle_mod.lora_epilogue(acc2, np.array([0.5], np.float32), np.array([0.25, 0.25], np.float32),
                                  xa, b, 0.25)
    assert y2.tolist() == _bf16([[12.5, 14.0]]).tolist()


def test_lora_epilogue_scale_power_of_two_invariance(oracle_mod):
    # scale * B == (2 scale) * (B / 2) exactly when B / 2 stays a normal bf16
    g = np.random.default_rng(5)
    acc = g.integers(-30000, 30000, (4, 6), dtype=np.int32)
    sx = (g.random(4) + 0.1).astype(np.float32) * 1e-3
    sw = (g.random(6) + 0.1).astype(np.float32) * 1e-3
    xa = _bf16(g.standard_normal((4, 32)))
    bf = wl.bf16_bits_to_f32(_bf16(g.standard_normal((6, 32))))
    y1 = oracle_mod.lora_epilogue(acc, sx, sw, xa, _bf16(bf), 0.375)
    y2 = oracle_mod.lora_epilogue(acc, sx, sw, xa, _bf16(bf / 2), 0.75)
    assert np.array_equal(y1, y2)
