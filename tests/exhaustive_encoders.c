/* Exhaustive check of the oracle's E2M1 and E4M3 encoders against brute-force
 * nearest-value searches written here from the format definitions.
 *
 *  E2M1: every fp32 bit pattern except NaN. Brute force: distance to each of
 *        the 8 grid magnitudes, the smallest wins, equal distances go to the
 *        even index; sign bit copied from the input.
 *  E4M3: every non-negative finite fp32 pattern. Brute force: the sorted list
 *        of the 127 finite non-negative E4M3 values (built from the bit
 *        layout), bisect for the neighbours, nearer wins, ties to the even
 *        byte; inputs at or above 448 give 0x7E.
 * Argument 2 = "fast": every pattern whose magnitude lies in the binades
 * where the code can change (E2M1: [2^-4, 2^4); E4M3: [2^-12, 2^10)), and
 * every 61st pattern elsewhere. "full" walks every pattern.
 * Prints "OK <counts>" or the first mismatch, exits non-zero on failure. */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

extern uint32_t orc_e2m1_encode(float y);
extern uint32_t orc_e4m3_encode(float v);

static const double grid[8] = {0, 0.5, 1, 1.5, 2, 3, 4, 6};
static double e4m3[127];

static uint32_t bf_e2m1(float y) {
  /* Beyond 6 the nearest grid value is 6; clamping keeps distances exact. */
  double a = fmin(fabs((double)y), 7.0);
  int best = 0;
  double bd = fabs(a - grid[0]);
  for (int i = 1; i < 8; ++i) {
    double d = fabs(a - grid[i]);
    if (d < bd || (d == bd && (i % 2 == 0) && (best % 2 == 1))) { bd = d; best = i; }
  }
  return (uint32_t)best | (signbit(y) ? 8u : 0u);
}

static uint32_t bf_e4m3(float v) {
  double x = (double)v;
  if (x >= 448.0) return 0x7E;
  int lo = 0, hi = 126; /* e4m3[lo] <= x < e4m3[hi] */
  while (hi - lo > 1) {
    int mid = (lo + hi) / 2;
    if (e4m3[mid] <= x) lo = mid; else hi = mid;
  }
  double dl = x - e4m3[lo], dh = e4m3[hi] - x;
  if (dl < dh) return (uint32_t)lo;
  if (dh < dl) return (uint32_t)hi;
  return (lo % 2 == 0) ? (uint32_t)lo : (uint32_t)hi;
}

typedef struct { uint64_t begin, end; int which, fast; uint64_t bad, n; uint32_t first_bad; } job_t;

static int dense_region(int which, uint32_t b) {
  uint32_t e = (b >> 23) & 0xFFu; /* biased exponent */
  return which == 0 ? (e >= 123u && e < 131u) : (e >= 115u && e < 137u);
}

static void* run(void* p) {
  job_t* j = (job_t*)p;
  for (uint64_t u = j->begin; u < j->end; ++u) {
    uint32_t b = (uint32_t)u;
    float f;
    memcpy(&f, &b, 4);
    if (isnan(f)) continue;
    if (j->fast && !dense_region(j->which, b) && (u % 61u) != 0) continue;
    if (j->which == 1 && (signbit(f) || isinf(f))) continue;
    uint32_t a = j->which == 0 ? orc_e2m1_encode(f) : orc_e4m3_encode(f);
    uint32_t e = j->which == 0 ? bf_e2m1(f) : bf_e4m3(f);
    j->n++;
    if (a != e) { if (!j->bad) j->first_bad = b; j->bad++; }
  }
  return NULL;
}

int main(int argc, char** argv) {
  int nthreads = argc > 1 ? atoi(argv[1]) : 8;
  int fast = argc > 2 && strcmp(argv[2], "fast") == 0;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 64) nthreads = 64;
  for (int b = 0; b < 127; ++b) {
    int e = b >> 3, m = b & 7;
    e4m3[b] = e ? ldexp(1.0 + m / 8.0, e - 7) : ldexp(m / 8.0, -6);
  }
  int fail = 0;
  for (int which = 0; which < 2; ++which) {
    uint64_t total = which == 0 ? (1ull << 32) : 0x7F800000ull;
    pthread_t th[64];
    job_t jobs[64];
    for (int t = 0; t < nthreads; ++t) {
      jobs[t].begin = total * t / nthreads;
      jobs[t].end = total * (t + 1) / nthreads;
      jobs[t].which = which; jobs[t].fast = fast; jobs[t].bad = 0; jobs[t].n = 0; jobs[t].first_bad = 0;
      pthread_create(&th[t], NULL, run, &jobs[t]);
    }
    uint64_t bad = 0, n = 0; uint32_t first = 0;
    for (int t = 0; t < nthreads; ++t) {
      pthread_join(th[t], NULL);
      if (jobs[t].bad && !bad) first = jobs[t].first_bad;
      bad += jobs[t].bad; n += jobs[t].n;
    }
    printf("%s checked %llu mismatches %llu first 0x%08x\n", which ? "e4m3" : "e2m1",
           (unsigned long long)n, (unsigned long long)bad, first);
    if (bad) fail = 1;
  }
  printf(fail ? "FAIL\n" : "OK\n");
  return fail;
}
