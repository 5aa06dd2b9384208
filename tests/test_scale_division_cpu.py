"""The block-scale divisions of the kernels against IEEE division, checked
on the CPU in binary32 (gcc, fmaf): the kernels compute amax / Qmax by
Markstein's correction around the constant RN(1/Qmax), and 1/s by one Newton
step from the hardware reciprocal, for scales stored as fp16 or E4M3.

- Reciprocal: for every positive finite fp16 value and every positive E4M3
  value s, each start r0 within 4 ulp of 1/s ends on RN(1/s) after
  r0 + r0 * (1 - s * r0) with fused operations (exhaustive). v_rcp_f32 is
  within 1 ulp.
- Quotient: for each format's Qmax, every binary32 amax of eleven exponent
  bands (all significands of each band, the tiny end among them) gives the
  IEEE quotient wherever that is at least 2^-125. Below, the quotient rounds
  to a zero fp16 or E4M3 scale either way, so only the side of 2^-126 it
  falls on is compared.
"""
import os
import subprocess
import tempfile

import pytest

SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static int recip_ok(float s) {
  const float rn = 1.0f / s;
  for (int k = -4; k <= 4; k++) {
    const float r0 = f_of(u_of(rn) + (uint32_t)k);
    const float r = fmaf(fmaf(-s, r0, 1.0f), r0, r0);
    if (r != rn) return 0;
  }
  return 1;
}

int main(void) {
  long bad = 0, n = 0;
  for (uint32_t h = 1; h < 0x7C00; h++) {            /* fp16 positive finite */
    const int e = (h >> 10) & 31, m = h & 1023;
    const float s = e == 0 ? ldexpf((float)m, -24) : ldexpf((float)(1024 + m), e - 25);
    bad += !recip_ok(s); n++;
  }
  for (int e = 0; e < 16; e++)                       /* E4M3 positive finite */
    for (int m = 0; m < 8; m++) {
      if ((e == 15 && m == 7) || (e == 0 && m == 0)) continue;
      const float s = e == 0 ? ldexpf((float)m / 8.0f, -6) : ldexpf(1.0f + (float)m / 8.0f, e - 7);
      bad += !recip_ok(s); n++;
    }
  printf("recip %ld %ld\n", n, bad);

  const float qs[7] = {127.f, 7.f, 448.f, 57344.f, 6.f, 7.5f, 28.f};
  const int bands[11] = {0, 1, 2, 3, 4, 40, 100, 127, 128, 200, 254};  /* biased exponents */
  const float lim = ldexpf(1.0f, -125);
  for (int qi = 0; qi < 7; qi++) {
    const float q = qs[qi];
    volatile float one = 1.0f;
    const float r = one / q;
    long mism = 0, tiny = 0, cnt = 0;
#pragma omp parallel for collapse(2) reduction(+ : mism, tiny, cnt) schedule(static)
    for (int b = 0; b < 11; b++)
      for (uint32_t m = 0; m < (1u << 23); m++) {
        const float a = f_of(((uint32_t)bands[b] << 23) | m);
        const float ieee = a / q;
        const float q0 = a * r;
        const float v = fmaf(-fmaf(q0, q, -a), r, q0);
        cnt++;
        if (v == ieee) continue;
        if (ieee >= lim) mism++;
        else { tiny++; if ((v >= ldexpf(1.0f, -126)) != (ieee >= ldexpf(1.0f, -126))) mism++; }
      }
    printf("qmax %g %ld %ld %ld\n", q, cnt, mism, tiny);
  }
  return 0;
}
"""


@pytest.fixture(scope="module")
def report():
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "div.c"), os.path.join(d, "div")
        with open(src, "w") as f:
            f.write(SRC)
        subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-o", exe, src, "-lm"], check=True)
        out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout
    return out.split("\n")


def test_newton_reciprocal_of_fp16_and_e4m3_scales(report):
    n, bad = map(int, report[0].split()[1:])
    assert n == 31743 + 126
    assert bad == 0


def test_markstein_scale_quotients(report):
    rows = [r.split() for r in report[1:] if r.startswith("qmax")]
    assert len(rows) == 7
    tiny_seen = 0
    for _, q, cnt, mism, tiny in rows:
        assert int(cnt) == 11 << 23, q
        assert int(mism) == 0, f"Qmax {q}: quotients >= 2^-125 differ from IEEE division"
        tiny_seen += int(tiny)
    assert tiny_seen > 0   # the differences below 2^-125 exist: the bands reach them
