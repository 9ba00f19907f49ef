/* The kernels' E4M3 block-scale step divides by 6 as q1 = fma(fma(-q0, 6, x),
 * y, q0) with q0 = RN(x * y), y = RN(1/6) (two fused multiply-adds instead
 * of a full division). This walks every finite fp32 x >= 0 and checks that
 * q1 is bit-identical to the correctly rounded x / 6, or that both lie below
 * 2^-120 (where the E4M3 encoding is byte 0 for either).
 * Compiled with -ffp-contract=off so that x * y stays one rounded product.
 * Prints "OK <count>" or the first mismatch, exits non-zero on failure. */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct { uint32_t begin, end; uint64_t bad, n; uint32_t first_bad; } job_t;

static void* run(void* p) {
  job_t* j = (job_t*)p;
  const float y = 0x1.555556p-3f, tiny = 0x1p-120f;
  for (uint32_t b = j->begin; b < j->end; ++b) {
    float x;
    memcpy(&x, &b, 4);
    const float q0 = x * y;
    const float q1 = fmaf(fmaf(-q0, 6.0f, x), y, q0);
    const float ref = x / 6.0f;
    uint32_t a, e;
    memcpy(&a, &q1, 4);
    memcpy(&e, &ref, 4);
    j->n++;
    if (a != e && !(ref < tiny && q1 < tiny)) {
      if (!j->bad) j->first_bad = b;
      j->bad++;
    }
  }
  return NULL;
}

int main(int argc, char** argv) {
  int nthreads = argc > 1 ? atoi(argv[1]) : 8;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 64) nthreads = 64;
  const uint64_t total = 0x7F800000ull; /* every finite non-negative pattern */
  pthread_t th[64];
  job_t jobs[64];
  for (int t = 0; t < nthreads; ++t) {
    jobs[t].begin = (uint32_t)(total * t / nthreads);
    jobs[t].end = (uint32_t)(total * (t + 1) / nthreads);
    jobs[t].bad = 0; jobs[t].n = 0; jobs[t].first_bad = 0;
    pthread_create(&th[t], NULL, run, &jobs[t]);
  }
  uint64_t bad = 0, n = 0;
  uint32_t first = 0;
  for (int t = 0; t < nthreads; ++t) {
    pthread_join(th[t], NULL);
    if (jobs[t].bad && !bad) first = jobs[t].first_bad;
    bad += jobs[t].bad;
    n += jobs[t].n;
  }
  if (bad) {
    printf("FAIL %llu mismatches, first x bits 0x%08x\n", (unsigned long long)bad, first);
    return 1;
  }
  printf("OK %llu\n", (unsigned long long)n);
  return 0;
}
