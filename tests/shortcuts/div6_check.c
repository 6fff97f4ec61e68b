/* div6_check.c - exhaustive check of the fast divide-by-6 used by the
 * NVFP4 block scale (a_b / 6) and the MBS-Static macro factor (a_M / 6)
 * ("Unveiling the Potential of Quantization with MXFP4", technical summary
 * sections 1 and 2.B).
 *
 * The kernels form fl32(a / 6) as q0 = fl(a * fl32(1/6)), then
 * fl(fma(fma(-q0, 6, a), fl32(1/6), q0)): one product and a residual
 * correction. This program compares that with IEEE single-precision division
 * for every non-negative fp32 bit pattern in [lo, hi] (default: from 2^-125,
 * where the quotient is still normal, to the largest finite value) and
 * prints the number of differences. Build: gcc -O2 -ffp-contract=off
 * (no fast-math), so that every operation is the IEEE one written.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  uint32_t lo, hi;
  uint64_t bad;
  uint32_t first_bad;
} job_t;

static float from_bits(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return f;
}
static uint32_t to_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}

static void *run(void *arg) {
  job_t *j = (job_t *)arg;
  const volatile float six = 6.0f;
  const float sixth = 1.0f / six; /* fl32(1/6), rounded at run time */
  j->bad = 0;
  j->first_bad = 0;
  for (uint64_t u = j->lo; u <= j->hi; u++) {
    const float a = from_bits((uint32_t)u);
    const float q0 = a * sixth;
    const float fast = fmaf(fmaf(-q0, 6.0f, a), sixth, q0);
    const float ieee = a / six;
    if (to_bits(fast) != to_bits(ieee)) {
      if (j->bad == 0) j->first_bad = (uint32_t)u;
      j->bad++;
    }
  }
  return NULL;
}

int main(int argc, char **argv) {
  uint32_t lo = argc > 1 ? (uint32_t)strtoul(argv[1], NULL, 0) : 0x01000000u;
  uint32_t hi = argc > 2 ? (uint32_t)strtoul(argv[2], NULL, 0) : 0x7F7FFFFFu;
  int threads = argc > 3 ? atoi(argv[3]) : 8;
  if (threads < 1 || threads > 64) threads = 8;
  pthread_t tid[64];
  job_t jobs[64];
  uint64_t n = (uint64_t)hi - lo + 1;
  for (int t = 0; t < threads; t++) {
    jobs[t].lo = (uint32_t)(lo + n * t / threads);
    jobs[t].hi = (uint32_t)(lo + n * (t + 1) / threads - 1);
    pthread_create(&tid[t], NULL, run, &jobs[t]);
  }
  uint64_t bad = 0;
  uint32_t first = 0;
  for (int t = 0; t < threads; t++) {
    pthread_join(tid[t], NULL);
    if (jobs[t].bad && !bad) first = jobs[t].first_bad;
    bad += jobs[t].bad;
  }
  printf("checked %llu patterns, %llu differ", (unsigned long long)n, (unsigned long long)bad);
  if (bad) printf(", first 0x%08x", first);
  printf("\n");
  return bad ? 1 : 0;
}
