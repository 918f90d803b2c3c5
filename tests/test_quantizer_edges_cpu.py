"""Edges of the per-row quantizer: subnormal and underflowing scales, and the
short quotient the kernels use.

Three kinds of check, none needing a GPU:

* oracle pins derived by hand for rows whose scale s = fl32(a / 127) is
  subnormal or zero (the int8 input gradient reaches such rows: the fold
  g = fl32(dY) * s_w can be far below any bf16 activation);
* a host emulation, in C, of the two branches of the kernels' per-row
  arithmetic (the 3-operation quotient for ordinary rows, the IEEE division
  with the clamp to +-127 for extreme ones), compared code for code with the
  oracle on crafted fold rows; the same emulation without the clamp is shown
  to disagree, so the rows do reach the case the clamp exists for;
* the kernels' correctly rounded quotient (Markstein's correction step with
  inv = RN(1/s)) against the IEEE quotient on adversarial pairs: exact
  half-integer quotients, their neighbours one ulp away, divisors with
  all-ones significands, every binade of s the kernels send through it.

Sources: "LoRA Training Guide for MOSS-Image", section 7.1, "ConvRot INT8" (the
opt-in int8 backward quantizes the gradient per row); scale = absmax / 127 and
round-half-to-even of the quotient, clamped to [-127, 127].
"""
import ctypes as C
import shutil
import subprocess

import numpy as np
import pytest

import workloads as wl
from crafted import nonfinite_fold_rows, nonfinite_rows, tiny_fold_rows

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")

P = 2.0 ** -149   # smallest fp32 subnormal


def f32(v):
    return np.asarray(v, dtype=np.float32)


# --------------------------------------------------------------------------
# Oracle pins (hand-derived)
# --------------------------------------------------------------------------

def test_subnormal_scale_clamps_the_maximum(oracle_mod):
    # a = 2^-140: a / 127 = 2^-149 * 512/127 = 4.031 * 2^-149, which rounds to
    # 4 * 2^-149 = 2^-147 (subnormal).  The quotients are then exact:
    # 2^-140 / 2^-147 = 128 (clamped to 127), 2^-141 / 2^-147 = 64,
    # -0.75 * 2^-140 / 2^-147 = -96, 2^-149 / 2^-147 = 0.25 -> 0.
    r = f32([[2.0 ** -140, 2.0 ** -141, -0.75 * 2.0 ** -140, P, 0.0, -2.0 ** -140]])
    q, s = oracle_mod.quantize_rows(r)
    assert float(s[0]) == 2.0 ** -147
    assert q[0].tolist() == [127, 64, -96, 0, 0, -127]


def test_scale_that_underflows_gives_zero_codes(oracle_mod):
    # a = 2^-144: a / 127 = 0.252 * 2^-149 < 2^-150, so s rounds to 0; the row
    # dequantizes to 0 whatever its codes, and they are 0 as for an all-zero row.
    r = f32([[2.0 ** -144, -2.0 ** -145, 0.0, P]])
    q, s = oracle_mod.quantize_rows(r)
    assert float(s[0]) == 0.0 and not q.any()


def test_smallest_nonzero_scale(oracle_mod):
    # a = 2^-143: a / 127 = 0.504 * 2^-149 rounds up to 2^-149, the smallest
    # subnormal; the maximum's code is then 2^-143 / 2^-149 = 64, not 127 (the
    # "absmax maps to 127" property needs a scale with a full significand).
    r = f32([[2.0 ** -143, -2.0 ** -144, 3 * P]])
    q, s = oracle_mod.quantize_rows(r)
    assert float(s[0]) == P
    assert q[0].tolist() == [64, -32, 3]


def test_fold_reaches_the_subnormal_scale(oracle_mod):
    # dY = 2^-120 (bf16 normal) and s_w = 2^-20 fold to g = 2^-140: the same row
    # as the first pin, reached through the int8 input gradient's quantizer.
    dy = wl.f32_to_bf16_bits(f32([[2.0 ** -120, 2.0 ** -121, -0.75 * 2.0 ** -120, 0.0]]))
    sw = f32([2.0 ** -20] * 4)
    q, s = oracle_mod.bwd_quant_dy(dy, sw)
    assert float(s[0]) == 2.0 ** -147
    assert q[0].tolist() == [127, 64, -96, 0]


# --------------------------------------------------------------------------
# Host emulation of the kernels' per-row branches
# --------------------------------------------------------------------------

EMU_SRC = r"""
#include <math.h>
#include <stdint.h>
#include <string.h>

static float bf16f(uint16_t b) { uint32_t u = (uint32_t)b << 16; float f; memcpy(&f, &u, 4); return f; }
static float quot_rn(float r, float s, float inv) {
  float q0 = r * inv;
  float e = fmaf(-q0, s, r);
  return fmaf(e, inv, q0);
}
/* low byte of t + 1.5 * 2^23: round half to even of |t| < 2^22 */
static int8_t low_byte(float t) {
  float v = t + 12582912.0f; uint32_t u; memcpy(&u, &v, 4); return (int8_t)(u & 0xff);
}

/* The fold quantizer of the int8 input gradient, as the kernels evaluate it:
   r = fl32(dY) * s_w; m = max |r| under the NaN-propagating maximum; ordinary
   rows (m in [2^-64, 2^100]) take s = quot_rn(m, 127, RN(1/127)) and
   t = quot_rn(r, s, RN(1/s)); other rows take the IEEE divisions, t clamped to
   [-127, 127] when clamp != 0, codes 0 when s == 0; a non-finite m gives the
   canonical NaN scale (and, since s > 0 fails, codes 0). */
static float max_nan(float a, float b) { return (isnan(a) || isnan(b)) ? NAN : fmaxf(a, b); }
static float nan_scale(void) { uint32_t u = 0x7fc00000u; float f; memcpy(&f, &u, 4); return f; }
void emu_fold(const uint16_t* dy, int64_t M, int64_t N, const float* sw, int clamp,
              int8_t* q, float* s_out) {
  const float y127 = 0x1.020408p-7f;
  for (int64_t m = 0; m < M; ++m) {
    float mx = 0.f;
    for (int64_t n = 0; n < N; ++n) mx = max_nan(mx, fabsf(bf16f(dy[m * N + n]) * sw[n]));
    float s;
    int fast = mx >= 0x1p-64f && mx <= 0x1p100f;
    if (fast) s = quot_rn(mx, 127.0f, y127);
    else s = mx <= 0x1.fffffep127f ? mx / 127.0f : nan_scale();
    float inv = s > 0.f ? 1.0f / s : 0.f;
    for (int64_t n = 0; n < N; ++n) {
      float r = bf16f(dy[m * N + n]) * sw[n], t;
      if (fast) t = quot_rn(r, s, inv);
      else if (s > 0.f) { t = r / s; if (clamp) t = fminf(fmaxf(t, -127.0f), 127.0f); }
      else t = 0.f;
      q[m * N + n] = low_byte(t);
    }
    s_out[m] = s;
  }
}

/* quot_rn against the IEEE quotient on n pairs; returns the number of pairs
   whose results differ (bit patterns), and the first differing index in *first. */
int64_t quot_check(const float* r, const float* s, int64_t n, int64_t* first) {
  int64_t bad = 0;
  *first = -1;
  for (int64_t i = 0; i < n; ++i) {
    volatile float ref = r[i] / s[i];
    float inv = 1.0f / s[i];
    float t = quot_rn(r[i], s[i], inv);
    uint32_t a, b; float rr = ref;
    memcpy(&a, &t, 4); memcpy(&b, &rr, 4);
    if (a != b) { if (bad == 0) *first = i; ++bad; }
  }
  return bad;
}
"""


@pytest.fixture(scope="module")
def emu(tmp_path_factory):
    d = tmp_path_factory.mktemp("emu")
    src, so = d / "emu.c", d / "libemu.so"
    src.write_text(EMU_SRC)
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-shared", "-fPIC",
                    "-o", str(so), str(src), "-lm"], check=True, capture_output=True)
    L = C.CDLL(str(so))
    p, i64 = C.c_void_p, C.c_int64
    L.emu_fold.argtypes = [p, i64, i64, p, C.c_int, p, p]
    L.quot_check.argtypes = [p, p, i64, C.POINTER(C.c_int64)]
    L.quot_check.restype = i64
    return L


def _ptr(a):
    return a.ctypes.data_as(C.c_void_p)


def emu_fold(L, dy, sw, clamp=True):
    dy = np.ascontiguousarray(dy, np.uint16)
    sw = np.ascontiguousarray(sw, np.float32)
    M, N = dy.shape
    q = np.empty((M, N), np.int8)
    s = np.empty(M, np.float32)
    L.emu_fold(_ptr(dy), M, N, _ptr(sw), int(clamp), _ptr(q), _ptr(s))
    return q, s


@pytest.mark.parametrize("N", [256, 2048, 4096])
def test_kernel_branches_match_the_oracle_on_tiny_fold_rows(oracle_mod, emu, N):
    dy, sw = tiny_fold_rows(N, N)
    if N == 4096:  # column scales that round the fold onto the subnormal grid
        sw = (np.random.default_rng(2).uniform(0.5, 1.0, N) * 2.0 ** -20).astype(np.float32)
    oq, os_ = oracle_mod.bwd_quant_dy(dy, sw)
    q, s = emu_fold(emu, dy, sw, clamp=True)
    assert np.array_equal(s.view(np.uint32), os_.view(np.uint32))
    assert np.array_equal(q, oq)
    # scales reach the subnormal range and zero
    assert (os_ == 0).any() and ((os_ > 0) & (os_ < 2.0 ** -126)).sum() >= 10
    # without the clamp the emulated kernel wraps quotients past 127.5 into
    # negative bytes (-128 for t = 128; a subnormal s can be off by far more, up
    # to t ~ 190) where the oracle has +-127
    q2, _ = emu_fold(emu, dy, sw, clamp=False)
    diff = q2 != oq
    assert diff.any()
    assert set(np.unique(np.abs(oq[diff].astype(np.int32))).tolist()) == {127}
    assert (q2[diff] == -128).any()


def test_kernel_branches_match_the_oracle_on_ordinary_rows(oracle_mod, emu):
    # the 3-operation path on ordinary gradients, crafted ties and huge/tiny scales
    dy = wl.normal_bf16((64, 1152), wl.SIGMA_DY, 5, 3)
    sw = (np.random.default_rng(1).random(1152) * 1e-3 + 1e-5).astype(np.float32)
    oq, os_ = oracle_mod.bwd_quant_dy(dy, sw)
    q, s = emu_fold(emu, dy, sw)
    assert np.array_equal(s.view(np.uint32), os_.view(np.uint32))
    assert np.array_equal(q, oq)


def test_kernel_branches_match_the_oracle_on_nonfinite_rows(oracle_mod, emu):
    # a NaN or infinite fold: the NaN-propagating maximum sends the row to the
    # NaN scale with codes 0 in the emulated kernel and in the oracle alike
    dy, sw = nonfinite_fold_rows(1152, 4)
    oq, os_ = oracle_mod.bwd_quant_dy(dy, sw)
    q, s = emu_fold(emu, dy, sw)
    assert np.array_equal(s.view(np.uint32), os_.view(np.uint32))
    assert np.array_equal(q, oq)
    assert (os_[:4].view(np.uint32) == NAN_BITS).all() and not oq[:4].any()
    assert np.isfinite(os_[4]) and os_[4] > 0


# --------------------------------------------------------------------------
# Non-finite rows (oracle pins)
# --------------------------------------------------------------------------

NAN_BITS = 0x7FC00000


def test_nonfinite_values_give_the_nan_scale(oracle_mod):
    # NaN, +inf, -inf anywhere in a row: scale = the canonical quiet NaN, codes
    # 0 (the row dequantizes to NaN); a finite row in the same call is untouched
    r = f32([[1.0, np.nan, -2.0, 0.5], [1.0, np.inf, -2.0, 0.5], [-np.inf, 3.0, 0.0, 1.0],
             [1.0, 4.0, -2.0, 0.5]])
    q, s = oracle_mod.quantize_rows(r)
    assert (s[:3].view(np.uint32) == NAN_BITS).all()
    assert not q[:3].any()
    q3, s3 = oracle_mod.quantize_rows(r[3:])
    assert s[3] == s3[0] and np.array_equal(q[3], q3[0]) and q3[0, 1] == 127


def test_rotation_of_nonfinite_rows(oracle_mod):
    # every crafted row is non-finite after the rotation (a NaN, +-inf, an
    # inf - inf block, an fp32 overflow of a block of bf16's largest value);
    # the last row is ordinary and keeps a finite scale
    for K in (128, 256, 4096):
        x = nonfinite_rows(K, K)
        q, s, _ = oracle_mod.rotate_quantize(x)
        assert (s[:6].view(np.uint32) == NAN_BITS).all(), K
        assert not q[:6].any(), K
        assert np.isfinite(s[6]) and s[6] > 0, K


def test_rotated_overflow_is_nonfinite(oracle_mod):
    # a block of 128 copies of bf16's largest value v: the rotated DC value is
    # fl32(128 v / sqrt(128)) = fl32(11.3 v) = +inf; the other 127 are 0
    v = 0x7F7F
    x = np.full((1, 128), v, np.uint16)
    r, _ = oracle_mod.rotate_rows(x)
    assert np.isinf(r[0, 0]) and not r[0, 1:].any()
    q, s, _ = oracle_mod.rotate_quantize(x)
    assert s.view(np.uint32)[0] == NAN_BITS and not q.any()


# --------------------------------------------------------------------------
# quot_rn against IEEE division
# --------------------------------------------------------------------------

def adversarial_pairs(seed: int = 0):
    """(r, s) pairs on which a quotient off by one ulp would change a code or a
    scale: for divisors s in every binade of [2^-64/127, 2^100/127] with short,
    all-ones and random significands, numerators r = (k + 1/2) * s (exact
    half-integer quotients, representable because s has at most 15 significant
    bits), their fp32 neighbours, and random r with |r| <= 127.5 * s."""
    g = np.random.default_rng(seed)
    rs, ss = [], []
    sig_short = [1.0, 1.5, 1.25, 1.75, 1.0 + 2.0 ** -14, 2.0 - 2.0 ** -14]
    for e in range(-71, 94):   # s from 2^-71 (< 2^-64 / 127) to 2^94 (> 2^100 / 127)
        sigs = list(sig_short)
        sigs.append(float(np.float32(2.0 - 2.0 ** -23)))          # all-ones significand
        sigs += [float(np.float32(1.0 + x)) for x in g.random(4)]  # random significands
        for sig in sigs:
            s = np.float32(sig * 2.0 ** e)
            k = np.arange(-128, 128, dtype=np.float64)
            if sig in sig_short:
                t = (k + 0.5)
                r = (t * np.float64(s)).astype(np.float32)     # exact
                assert np.all(r.astype(np.float64) == t * np.float64(s))
                up = np.nextafter(r, np.float32(np.inf))
                dn = np.nextafter(r, np.float32(-np.inf))
                cand = np.concatenate([r, up, dn])
            else:
                cand = (g.uniform(-127.5, 127.5, 256) * np.float64(s)).astype(np.float32)
                # numerators nearest to the half-integer quotients
                cand = np.concatenate([cand, ((k + 0.5) * np.float64(s)).astype(np.float32)])
            rs.append(cand)
            ss.append(np.full(cand.size, s, np.float32))
    return np.concatenate(rs), np.concatenate(ss)


def test_short_quotient_is_correctly_rounded(emu):
    r, s = adversarial_pairs()
    assert r.size > 500_000
    first = C.c_int64(-1)
    bad = emu.quot_check(_ptr(r), _ptr(s), r.size, C.byref(first))
    assert bad == 0, f"{bad} pairs differ, first r={r[first.value]!r} s={s[first.value]!r}"
