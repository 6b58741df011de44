"""Host check of the quotient shortcut used by the rotate + quantise kernel.

The kernel forms fl32(y / s) as q = fl32(y * r), rem = fma(-s, q, y),
fl32(q + rem * r) with r = fl32(1 / s) (Markstein's correction for binary32,
round to nearest) whenever s >= 2^-64, and the code is rne of that quotient.
This test compiles the same three float32 operations in C (gcc, no
contraction, libm fmaf) and compares them with the IEEE quotient on seeded
pairs drawn the way quantiser inputs occur: |y| <= qmax * s, quotients next
to k + 1/2, and s = fl32(amax / qmax).  Any differing quotient fails.
"""
import os
import shutil
import subprocess
import tempfile

import pytest

C_SRC = r"""
#include <stdio.h>
#include <stdint.h>
#include <math.h>
#include <string.h>
static uint64_t st = 88172645463325252ULL;
static uint64_t xr(void){ st ^= st << 13; st ^= st >> 7; st ^= st << 17; return st; }
static float u2f(uint32_t u){ float f; memcpy(&f,&u,4); return f; }
static uint32_t f2u(float f){ uint32_t u; memcpy(&u,&f,4); return u; }
int main(int argc, char **argv){
  long iters = atol(argv[1]), bad = 0, n = 0;
  for (long it = 0; it < iters; ++it) {
    int ex = (int)(xr() % 129) - 64;
    float s = ldexpf(1.0f + (float)(xr() & 0x7FFFFF) / 8388608.0f, ex);
    float qmax = (xr() & 1) ? 127.f : 7.f;
    float y;
    uint64_t mode = xr() % 4;
    if (mode == 0) {
      int k = (int)(xr() % 255) - 127;
      y = (k + 0.5f) * s;
      uint32_t u = f2u(y); u += (int)(xr() % 5) - 2; y = u2f(u);
    } else if (mode == 1) {
      double t = ((double)(xr() >> 11) / 9007199254740992.0) * 2 - 1;
      y = (float)(t * qmax * s);
    } else if (mode == 2) {
      y = ldexpf(1.0f + (float)(xr() & 0x7FFFFF) / 8388608.0f, ex + 7);
      s = y / qmax;
    } else {
      y = ldexpf(1.0f + (float)(xr() & 0x7FFFFF) / 8388608.0f, ex + (int)(xr() % 8) - 30) * ((xr() & 1) ? 1 : -1);
    }
    if (!(s >= 0x1p-64f) || !isfinite(y)) continue;
    float ref = y / s;
    float r = 1.0f / s;
    float q = y * r;
    float rem = fmaf(-s, q, y);
    float q2 = fmaf(rem, r, q);
    ++n;
    if (f2u(ref) != f2u(q2)) ++bad;
  }
  printf("%ld %ld\n", n, bad);
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_reciprocal_correction_equals_ieee_quotient():
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "q.c")
        exe = os.path.join(d, "q")
        with open(src, "w") as f:
            f.write(C_SRC.replace("#include <string.h>", "#include <string.h>\n#include <stdlib.h>"))
        subprocess.run(["gcc", "-O2", "-ffp-contract=off", src, "-o", exe, "-lm"], check=True)
        out = subprocess.run([exe, "20000000"], check=True, capture_output=True, text=True).stdout
    n, bad = map(int, out.split())
    assert n > 15_000_000
    assert bad == 0
