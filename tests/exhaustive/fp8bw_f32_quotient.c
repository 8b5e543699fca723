// Exhaustive check over the blockwise FP8 binary32-scale domain: for every
// positive finite BF16 block maximum a with s = RN32(a / 448) >= 2^-80 and
// every BF16 x with |x| <= a (both signs, -0 included), the signed E4M3 RNE
// code (saturating at 448) of RN32(x / s) equals that of
// copysign(fma(fma(-q0, s, x), r, q0), x), r = RN32(1 / s), q0 = RN32(x * r).
// Also counts bitwise differences of the quotients.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
static float bf(uint32_t b) { uint32_t u = b << 16; float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static double grid[127];
static int e4m3_mag(double q);
static int e4m3(float qf) {            // signed code: sign bit 7, RNE magnitude below
  const float c = fminf(fmaxf(qf, -448.0f), 448.0f);
  return e4m3_mag(fabs((double)c)) | (signbit(c) ? 0x80 : 0);
}
static int e4m3_mag(double q) {        // RNE onto the E4M3 magnitudes 0..448, saturating
  int lo = 0, hi = 126;
  while (hi - lo > 1) { int mid = (lo + hi) / 2; if (grid[mid] <= q) lo = mid; else hi = mid; }
  if (q >= grid[126]) return 126;
  double dl = q - grid[lo], dh = grid[hi] - q;
  if (dl < dh) return lo;
  if (dh < dl) return hi;
  return (lo & 1) ? hi : lo;
}
int main(void) {
  for (int c = 0; c < 127; ++c) {
    int e = c >> 3, m = c & 7;
    grid[c] = e == 0 ? m * ldexp(1.0, -9) : (1.0 + m / 8.0) * ldexp(1.0, e - 7);
  }
  long long pairs = 0, badcode = 0, badbits = 0, direct = 0;
  for (uint32_t ab = 1; ab < 0x7F80; ++ab) {
    const float a = bf(ab);
    const float s = a / 448.0f;
    if (s < 0x1p-80f) { ++direct; continue; }
    const float r = 1.0f / s;
    for (uint32_t k = 0; k <= 2 * ab + 1; ++k) {       // x and -x for every |x| <= a
      const uint32_t xb = (k >> 1) | ((k & 1) << 15);
      const float x = bf(xb);
      const float q = x / s;
      const float q0 = x * r;
      const float q1 = copysignf(fmaf(fmaf(-q0, s, x), r, q0), x);
      ++pairs;
      if (bits(q) != bits(q1)) ++badbits;
      if (e4m3(q) != e4m3(q1)) {
        if (badcode < 10) printf("code mismatch a=%a x=%a s=%a q=%a q1=%a\n", a, x, s, q, q1);
        ++badcode;
      }
    }
  }
  printf("pairs %lld code mismatches %lld quotient bit mismatches %lld maxima divided directly %lld\n",
         pairs, badcode, badbits, direct);
  return badcode != 0;
}
