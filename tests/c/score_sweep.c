/* Test helper: accuracy sweep of the oracle's pinned binary32 sigmoid against
 * the binary64 sigmoid 1/(1+exp(-x)) from libm, over ranges of binary32 bit
 * patterns.  Compiled by the test together with oracle/moe_oracle.c. */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <omp.h>

float orc_score(float x);

static float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* ulp of the binary32 grid at |v| (v > 0, normal range) */
static double ulp32(double v)
{
    int e;
    frexp(v, &e);          /* v = m 2^e, 0.5 <= m < 1 */
    return ldexp(1.0, e - 24);
}

/* Visits bit patterns lo, lo+step, ... <= hi.  out[0] = max error in ulps,
 * out[1] = the x where it occurs, out[2] = number of adjacent visited pairs
 * where S decreases as x increases, out[3] = number of values visited. */
void sweep(uint32_t lo, uint32_t hi, uint32_t step, double* out)
{
    double best = 0.0, bestx = 0.0, nonmono = 0.0, count = 0.0;
#pragma omp parallel
    {
        double b = 0.0, bx = 0.0, nm = 0.0, c = 0.0;
#pragma omp for schedule(static)
        for (int64_t u = lo; u <= (int64_t)hi; u += step) {
            float x = from_bits((uint32_t)u);
            double xd = (double)x;
            double ref = 1.0 / (1.0 + exp(-xd));
            float s = orc_score(x);
            double err = fabs((double)s - ref) / ulp32(ref);
            if (err > b) { b = err; bx = xd; }
            if ((int64_t)u + step <= (int64_t)hi) {
                float x2 = from_bits((uint32_t)(u + step));
                float s2 = orc_score(x2);
                /* ascending x means s2 >= s */
                if ((x2 > x && s2 < s) || (x2 < x && s2 > s)) nm += 1.0;
            }
            c += 1.0;
        }
#pragma omp critical
        {
            if (b > best) { best = b; bestx = bx; }
            nonmono += nm;
            count += c;
        }
    }
    out[0] = best; out[1] = bestx; out[2] = nonmono; out[3] = count;
}
