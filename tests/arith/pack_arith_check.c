/* CPU check of two IEEE binary32 identities the GPU Q8_0 pack kernel relies on (test
 * infrastructure; plain C, no GPU).
 *
 * 1. div127: for every finite a >= 0, q0 = RN(a * y) with y = RN(1/127), r = fma(-q0, 127, a)
 *    and d = fma(r, y, q0) give d = RN(a / 127).  Checked for all 2^31 - 2^23 such values.
 *
 * 2. The fast quantiser: for a normal FP16 scale dh (2^-14 <= dh <= 65504) and any reciprocal
 *    rdh within 2^-23 relative of 1/dh (the hardware reciprocal's bound), f = fma(x, rdh, M)
 *    with M = 1.5 * 2^23 and d = fma(x, rdh, M - f) give the integer r = f - M, and whenever
 *    |d| < 1/2 - 2^-13, r equals round(RN(x / dh)) with halves away from zero, clamped to
 *    [-127, 127], and the low byte of f's bits is r as a two's-complement byte.  Checked for
 *    every normal FP16 scale, three reciprocals (RN(1/dh) and one FP32 ulp either side), and for
 *    each integer k in [-127, 127] the inputs x within 3 ulps of k * dh, of (k + 1/2) * dh and of
 *    the window's edges (k + 1/2 -+ 2^-13) * dh that the scale's block can hold
 *    (|x| <= 127 * dh * (1 + 2^-11)).
 *
 * Prints "mismatches A B" (the counts of the two checks) and exits 0 when both are zero. */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#define NT 8

static float f_of(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }
static uint32_t b_of(float f) { uint32_t b; memcpy(&b, &f, 4); return b; }

typedef struct { int t; uint64_t bad1, bad2; } job_t;

static void *run(void *p)
{
    job_t *j = p;
    const float y = 1.0f / 127.0f;
    /* 1: interleaved 64 Ki-value slices so that the slow subnormal range is shared */
    for (uint64_t s = (uint64_t)j->t << 16; s < 0x7f800000u; s += (uint64_t)NT << 16) {
        for (uint64_t u = s; u < s + 65536 && u < 0x7f800000u; ++u) {
            const float a = f_of((uint32_t)u);
            volatile float ref = a / 127.0f;
            const float q0 = a * y;
            const float r = fmaf(-q0, 127.0f, a);
            const float d = fmaf(r, y, q0);
            if (b_of(d) != b_of(ref))
                j->bad1++;
        }
    }
    /* 2: FP16 exponent field 1..30, every mantissa */
    const float M = 0x1.8p23f;
    for (uint32_t h = 0x0400u + (uint32_t)j->t; h < 0x7c00u; h += NT) {
        const int e = (int)(h >> 10) - 15;
        const float dh = ldexpf(1.0f + (float)(h & 0x3ff) / 1024.0f, e);
        const float lim = 127.0f * dh * (1.0f + 0x1p-11f);
        const float rn = 1.0f / dh;
        const float rdhs[3] = {nextafterf(rn, 0.0f), rn, nextafterf(rn, INFINITY)};
        for (int k = -127; k <= 127; ++k) {
            for (int half = 0; half < 4; ++half) {
                /* k dh and (k + 1/2) dh (exact: at most 9 bits times 11), and the edges of the
                 * window, (k + 1/2 -+ 2^-13) dh rounded to FP32 */
                const double off[4] = {0.0, 0.5, 0.5 - 0x1p-13, 0.5 + 0x1p-13};
                const float c = (float)(((double)k + off[half]) * (double)dh);
                float x = c;
                for (int i = 0; i < 3; ++i)
                    x = nextafterf(x, -INFINITY);
                for (int i = 0; i < 7; ++i, x = nextafterf(x, INFINITY)) {
                    if (fabsf(x) > lim)
                        continue;
                    volatile float z = x / dh;
                    const float az = fabsf(z);
                    float q = truncf(az) + ((az - truncf(az)) >= 0.5f ? 1.0f : 0.0f);
                    q = fminf(q, 127.0f);
                    const int want = (int)copysignf(q, z);
                    for (int ri = 0; ri < 3; ++ri) {
                        const float rdh = rdhs[ri];
                        const float f = fmaf(x, rdh, M);
                        const float d = fmaf(x, rdh, M - f);
                        if (!(fabsf(d) < 0.5f - 0x1p-13f))
                            continue; /* the kernel's exact path takes this value */
                        const int r = (int)(f - M);
                        const uint8_t byte = (uint8_t)(b_of(f) & 0xffu);
                        if (r != want || byte != (uint8_t)(int8_t)want)
                            j->bad2++;
                    }
                }
            }
        }
    }
    return 0;
}

int main(void)
{
    pthread_t th[NT];
    job_t jb[NT];
    for (int t = 0; t < NT; ++t) {
        jb[t].t = t;
        jb[t].bad1 = jb[t].bad2 = 0;
        pthread_create(&th[t], 0, run, &jb[t]);
    }
    uint64_t b1 = 0, b2 = 0;
    for (int t = 0; t < NT; ++t) {
        pthread_join(th[t], 0);
        b1 += jb[t].bad1;
        b2 += jb[t].bad2;
    }
    printf("mismatches %llu %llu\n", (unsigned long long)b1, (unsigned long long)b2);
    return (b1 || b2) ? 1 : 0;
}
