/*
 * Independent checker for an fp32 -> OCP E4M3FN encoder (test helper).
 *
 * A code c is correct for y when: its sign bit equals y's; magnitudes >= 448
 * give 0x7E; otherwise the decoded value of c is at least as close to |y| as
 * the values of both neighbouring codes, and on an exact tie c is even.  This
 * characterisation is unique, so a code that passes is the nearest-even code.
 * The decoding here is written from the OCP 8-bit floating point format
 * (E4M3: bias 7, 3 mantissa bits, no infinities, S.1111.111 = NaN, subnormals
 * m * 2^-9), independently of the oracle's table.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC (see tests/test_oracle_pins.py).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

static double dec(int c)          /* non-negative codes 0..126 */
{
    int e = (c >> 3) & 15, m = c & 7;
    return e == 0 ? m * 0x1p-9 : (8 + m) * ldexp(1.0, e - 10);
}

static int ok(float y, uint8_t code)
{
    uint32_t b;
    memcpy(&b, &y, 4);
    if ((code >> 7) != (b >> 31)) return 0;
    int c = code & 0x7F;
    double a = fabs((double)y);
    if (a >= 448.0) return c == 0x7E;
    if (c == 0x7F) return 0;
    double v = dec(c), d = fabs(a - v);
    if (c > 0) {
        double dl = fabs(a - dec(c - 1));
        if (dl < d) return 0;
        if (dl == d && (c & 1)) return 0;
    }
    if (c < 126) {
        double dh = fabs(a - dec(c + 1));
        if (dh < d) return 0;
        if (dh == d && (c & 1)) return 0;
    }
    return 1;
}

typedef uint8_t (*enc_fn)(float);

/* Checks every fp32 bit pattern in [lo, hi) (non-NaN) with the encoder fn;
   returns the number of failures and stores the first failing pattern. */
int64_t check_fn(uint32_t lo, uint32_t hi, enc_fn fn, uint32_t* first_bad)
{
    int64_t bad = 0;
    uint32_t first = 0xFFFFFFFFu;
#pragma omp parallel for schedule(static, 1 << 16) reduction(+ : bad)
    for (int64_t i = lo; i < (int64_t)hi; ++i) {
        uint32_t bits = (uint32_t)i;
        float y;
        memcpy(&y, &bits, 4);
        if (isnan(y)) continue;
        if (!ok(y, fn(y))) {
            ++bad;
#pragma omp critical
            if (bits < first) first = bits;
        }
    }
    *first_bad = first;
    return bad;
}

/* Same, for codes already computed (e.g. by the GPU): codes[i] belongs to the
   pattern lo + i. */
int64_t check_codes(uint32_t lo, int64_t n, const uint8_t* codes, uint32_t* first_bad)
{
    int64_t bad = 0;
    uint32_t first = 0xFFFFFFFFu;
#pragma omp parallel for schedule(static, 1 << 16) reduction(+ : bad)
    for (int64_t i = 0; i < n; ++i) {
        uint32_t bits = lo + (uint32_t)i;
        float y;
        memcpy(&y, &bits, 4);
        if (isnan(y)) continue;
        if (!ok(y, codes[i])) {
            ++bad;
#pragma omp critical
            if (bits < first) first = bits;
        }
    }
    *first_bad = first;
    return bad;
}
