/*
 * Exhaustive pin of the oracle's E4M3 encoder over every binary32 bit
 * pattern (NaNs excluded: their code is undefined by the reading).
 *
 * The expected code is found by brute force, independently of the oracle's
 * bit construction: the 127 finite non-negative E4M3 values are generated
 * from the format definition (subnormals m*2^-9, normals (1+m/8)*2^e for
 * e = -6..8, capped at 448), sorted, and numbered in increasing order -- the
 * code of the i-th smallest magnitude is i because E4M3 stores magnitude as
 * exponent-above-mantissa.  A value maps to the nearest table entry, a tie to
 * the entry with the even number, and anything above 448 to 448; the sign
 * bit is 0x80.
 *
 * Usage: e4m3_exhaustive [threads]   -- prints "mismatches N" and exits 0
 * only when N == 0.
 */
#include "../../oracle/puro_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static double table[127];

static int cmp_d(const void* a, const void* b)
{
    double x = *(const double*)a, y = *(const double*)b;
    return (x > y) - (x < y);
}

static void build_table(void)
{
    int n = 0;
    for (int m = 0; m < 8; ++m)
        table[n++] = ldexp((double)m, -9);
    for (int e = -6; e <= 8; ++e)
        for (int m = 0; m < 8; ++m) {
            double v = (1.0 + m / 8.0) * ldexp(1.0, e);
            if (v <= 448.0)
                table[n++] = v;
        }
    if (n != 127) {
        fprintf(stderr, "table size %d\n", n);
        exit(2);
    }
    qsort(table, 127, sizeof(double), cmp_d);
}

static uint8_t brute(float v)
{
    uint32_t bits;
    memcpy(&bits, &v, 4);
    uint8_t sign = (bits >> 31) ? 0x80 : 0;
    double a = fabs((double)v);
    if (a > 448.0)
        return sign | 126;
    int lo = 0, hi = 126;              /* largest i with table[i] <= a */
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (table[mid] <= a) lo = mid; else hi = mid - 1;
    }
    int best = lo;
    if (lo < 126) {
        double dl = a - table[lo], dh = table[lo + 1] - a;
        if (dh < dl || (dh == dl && ((lo + 1) % 2 == 0)))
            best = lo + 1;
    }
    return sign | (uint8_t)best;
}

typedef struct { uint64_t begin, end, bad; uint32_t first_bad; } job;

static void* run(void* p)
{
    job* j = (job*)p;
    for (uint64_t u = j->begin; u < j->end; ++u) {
        uint32_t b = (uint32_t)u;
        float v;
        memcpy(&v, &b, 4);
        if (isnan(v))
            continue;
        if (orc_e4m3_encode(v) != brute(v)) {
            if (j->bad == 0) j->first_bad = b;
            j->bad++;
        }
    }
    return NULL;
}

int main(int argc, char** argv)
{
    int nt = argc > 1 ? atoi(argv[1]) : 8;
    if (nt < 1) nt = 1;
    if (nt > 64) nt = 64;
    build_table();
    pthread_t th[64];
    job jobs[64];
    const uint64_t total = 1ull << 32;
    for (int t = 0; t < nt; ++t) {
        jobs[t].begin = total * t / nt;
        jobs[t].end = total * (t + 1) / nt;
        jobs[t].bad = 0;
        jobs[t].first_bad = 0;
        pthread_create(&th[t], NULL, run, &jobs[t]);
    }
    uint64_t bad = 0;
    for (int t = 0; t < nt; ++t) {
        pthread_join(th[t], NULL);
        if (jobs[t].bad && !bad)
            fprintf(stderr, "first mismatch at bits 0x%08x\n", jobs[t].first_bad);
        bad += jobs[t].bad;
    }
    printf("mismatches %llu\n", (unsigned long long)bad);
    return bad == 0 ? 0 : 1;
}
