"""Host check of the short division the quantizer kernels use for the row scale.

The kernels form s = fl32(a / 127) with three fp32 operations (q0 = a*y,
e = fma(-q0, 127, a), s = fma(e, y, q0), y = RN(1/127)) whenever a lies in
[2^-64, 2^100], and with the IEEE division otherwise.  Scaling a by a power of
two scales every intermediate exactly in that range, so checking every fp32
significand of a in [1, 2) covers every such a.  This runs the sequence in C
with the C library's correctly rounded fmaf and compares it with the IEEE
quotient for all 2^23 significands.
"""
import shutil
import subprocess

import pytest

SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

int main(void) {
  const float y = 0x1.020408p-7f;            /* the constant the kernels use */
  volatile float one = 1.0f, d = 127.0f;
  if (y != one / d) { printf("y is not RN(1/127)\n"); return 2; }
  long bad = 0;
  for (uint32_t m = 0; m < (1u << 23); ++m) {
    uint32_t bits = (127u << 23) | m;
    float a;
    memcpy(&a, &bits, 4);
    volatile float ref = a / d;
    float q0 = a * y;
    float e = fmaf(-q0, 127.0f, a);
    float s = fmaf(e, y, q0);
    if (s != ref) ++bad;
  }
  printf("%ld\n", bad);
  return bad != 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_three_op_division_by_127_is_correctly_rounded(tmp_path):
    c = tmp_path / "q127.c"
    exe = tmp_path / "q127"
    c.write_text(SRC)
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", str(exe), str(c), "-lm"],
                   check=True, capture_output=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip() == "0"
