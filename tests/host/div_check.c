/* Exhaustive CPU check of the quotient used by the HIP quantizers.
 *
 * The kernels compute y = fl32(x / s) without a per-element IEEE division:
 * with r = fl32(1 / s) (one correctly rounded division per tile),
 *     y0 = fl32(x * r);  e = fma(-s, y0, x);  y = fma(e, r, y0)
 * and the sign of x copied onto y (x / s has the sign of x for s > 0).  This
 * is Markstein's FMA correction of a faithful quotient (P. Markstein, "Computation
 * of elementary functions on the IBM RISC System/6000 processor", IBM J. Res.
 * Dev. 34(1), 1990; J.-M. Muller et al., Handbook of Floating-Point Arithmetic,
 * the section on Newton-Raphson based division with an FMA).
 *
 * Every BF16 tile maximum amax > 0 gives one scale s = fl32(amax / 448); every
 * BF16 x with |x| <= amax can meet that s.  For each amax this program checks
 * all such x (both signs) and prints, as "FAIL <amax bits> <count>", every
 * amax for which the shortcut differs from x / s in a way that can change an
 * E4M3 code (any bit difference unless both values are at most 2^-10 with the
 * same sign).  The kernels use the
 * shortcut only for scales inside [2^-100, 2^100] (FAST_LO/FAST_HI), where
 * this check must report no failure; outside it they divide per element.
 *
 * Build: gcc -O2 -fopenmp -mfma -ffp-contract=off div_check.c -o div_check -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float f_of(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }
static uint32_t b_of(float f) { uint32_t b; memcpy(&b, &f, 4); return b; }

int main(int argc, char **argv) {
  const float FAST_LO = 0x1p-100f, FAST_HI = 0x1p100f;
  long long total_fail_fast = 0, total_checked = 0, slow_tiles = 0, tiny_diff = 0;
  #pragma omp parallel for schedule(dynamic, 64) reduction(+:total_fail_fast,total_checked,slow_tiles,tiny_diff)
  for (uint32_t ab = 1; ab < 0x7F80; ++ab) {          /* positive finite BF16 amax */
    const float amax = f_of(ab << 16);
    const float s = amax / 448.0f;
    if (!(s >= FAST_LO && s <= FAST_HI)) { slow_tiles++; continue; }
    const float r = 1.0f / s;
    long long fails = 0;
    for (uint32_t xb = 0; xb <= ab; ++xb) {
      for (int neg = 0; neg < 2; ++neg) {
        const float x = f_of((xb << 16) | (neg ? 0x80000000u : 0u));
        const float ref = x / s;
        const float y0 = x * r;
        const float e = fmaf(-s, y0, x);
        float y = fmaf(e, r, y0);
        y = copysignf(y, x);
        /* Below 2^-10 every value encodes to a signed zero in E4M3 (2^-10 is
         * the tie between 0 and the smallest subnormal 2^-9 and goes to the
         * even code 0), so a difference there cannot change a code; the
         * residual e underflows for such tiny x and y stays at y0. */
        const int same = b_of(y) == b_of(ref);
        const int both_zero_code = fabsf(y) <= 0x1p-10f && fabsf(ref) <= 0x1p-10f &&
                                   signbit(y) == signbit(ref);
        if (!same && !both_zero_code) fails++;
        if (!same) tiny_diff++;
        total_checked++;
      }
    }
    if (fails) {
      #pragma omp critical
      printf("FAIL %#06x %lld\n", ab, fails);
      total_fail_fast += fails;
    }
  }
  printf("checked %lld quotients, %lld code-relevant mismatches in the fast range, "
         "%lld harmless differences below 2^-10, %lld amax values use per-element division\n",
         total_checked, total_fail_fast, tiny_diff, slow_tiles);
  return total_fail_fast != 0;
}
