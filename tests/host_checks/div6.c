/* Host check of the device division by 6 used for the NVFP4 block scale: q0 = a * fl32(1/6),
 * q = fma(fma(-q0, 6, a), fl32(1/6), q0) must equal the correctly rounded fl32(a / 6) for every
 * finite fp32 a >= 2^-125 (bit patterns 0x01000000 .. 0x7F7FFFFF). The reference quotient is the
 * double quotient rounded to float (double has more than 2 * 24 + 2 bits, so that rounding twice
 * gives the correctly rounded fp32 quotient). Prints the number of mismatches. */
#include <stdio.h>
#include <stdint.h>
#include <string.h>
#include <math.h>

static float f_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t u_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

int main(void)
{
    const float c = (float)(1.0 / 6.0);
    long long bad = 0;
#pragma omp parallel for reduction(+ : bad) schedule(static)
    for (long long u = 0x01000000LL; u < 0x7F800000LL; ++u) {
        float a = f_of((uint32_t)u);
        float want = (float)((double)a / 6.0);
        float q0 = a * c;
        float q = fmaf(fmaf(-q0, 6.0f, a), c, q0);
        if (u_of(q) != u_of(want)) ++bad;
    }
    printf("%lld\n", bad);
    return 0;
}
