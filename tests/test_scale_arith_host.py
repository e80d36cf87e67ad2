"""Host check of an arithmetic identity the quantize kernels rely on.

The NVFP4 block scale starts with amax_b / 6 rounded to nearest even in FP32.
The kernels compute it, for amax_b >= 2^-100, as q0 = amax_b * RN(1/6) followed
by one fma correction q0 + RN(1/6) * (amax_b - 6 q0), and below 2^-100 by the
division itself. This test checks the identity for every FP32 value from
2^-100 to the largest finite one against the IEEE division (C's `/`, round to
nearest even), so that the kernels' scale bytes equal the oracle's for every
block amax, not only for the blocks the parity tests happen to contain."""
import os
import subprocess
import tempfile

SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
static float f(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }
static uint32_t b(float x) { uint32_t u; memcpy(&u, &x, 4); return u; }
int main(void) {
  const float r6 = 0x1.555556p-3f;            /* RN(1/6) */
  long bad = 0;
  #pragma omp parallel for reduction(+:bad) schedule(static)
  for (long i = 0x0D800000L; i < 0x7F800000L; ++i) {   /* 2^-100 .. FLT_MAX */
    const float m = f((uint32_t)i);
    const float q0 = m * r6;
    const float q = fmaf(fmaf(-6.0f, q0, m), r6, q0);
    if (b(q) != b(m / 6.0f)) bad++;
  }
  printf("%ld\n", bad);
  return 0;
}
"""


def test_div6_equals_ieee_division_from_2_pow_minus_100():
    assert 0x0D800000 == (127 - 100) << 23          # the bit pattern of 2^-100
    with tempfile.TemporaryDirectory() as d:
        c, exe = os.path.join(d, "div6.c"), os.path.join(d, "div6")
        with open(c, "w") as fh:
            fh.write(SRC)
        subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", c, "-o", exe, "-lm"],
                       check=True)
        out = subprocess.run([exe], capture_output=True, text=True, check=True, timeout=300).stdout
    assert out.strip() == "0"
