/*
 * Exhaustive check of binary16 directed rounding over every binary32 pattern.
 *
 * The functions under test are passed in as pointers (the oracle's
 * kvqr_rd16_n / kvqr_ru16_n).  The expected behaviour comes from tables the
 * test builds with numpy from its own binary16 decoder, never from the code
 * under test:
 *   val[h]  value of pattern h (NaN for NaN patterns),
 *   up[h]   next strictly larger binary16 value (+inf above 65504),
 *   down[h] next strictly smaller binary16 value (-inf below -65504).
 * Defining properties: rd = RD16(x) satisfies val[rd] <= x < up[rd];
 * ru = RU16(x) satisfies down[ru] < x <= val[ru]; +-inf map to themselves;
 * NaN maps to a NaN pattern.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef void (*round_fn)(const float*, int64_t, uint16_t*);

typedef struct {
  const double *val, *up, *down;
  round_fn rd, ru;
  uint64_t start, end;
  int64_t fails;
  uint32_t first_fail;
} job_t;

#define CHUNK (1 << 16)

static void* worker(void* arg) {
  job_t* j = (job_t*)arg;
  float* x = (float*)malloc(sizeof(float) * CHUNK);
  uint16_t* a = (uint16_t*)malloc(2 * CHUNK);
  uint16_t* b = (uint16_t*)malloc(2 * CHUNK);
  for (uint64_t s = j->start; s < j->end; s += CHUNK) {
    int64_t n = (int64_t)((j->end - s) < CHUNK ? (j->end - s) : CHUNK);
    for (int64_t i = 0; i < n; i++) {
      uint32_t u = (uint32_t)(s + (uint64_t)i);
      memcpy(&x[i], &u, 4);
    }
    j->rd(x, n, a);
    j->ru(x, n, b);
    for (int64_t i = 0; i < n; i++) {
      double xv = (double)x[i];
      int ok;
      if (isnan(xv)) {
        ok = isnan(j->val[a[i]]) && isnan(j->val[b[i]]);
      } else {
        /* at +-inf the value is exact: there is no neighbour beyond it */
        int rd_ok = (j->val[a[i]] <= xv) && (xv < j->up[a[i]] || (isinf(xv) && j->val[a[i]] == xv));
        int ru_ok = (xv <= j->val[b[i]]) && (j->down[b[i]] < xv || (isinf(xv) && j->val[b[i]] == xv));
        ok = rd_ok && ru_ok;
      }
      if (!ok) {
        if (j->fails == 0) j->first_fail = (uint32_t)(s + (uint64_t)i);
        j->fails++;
      }
    }
  }
  free(x);
  free(a);
  free(b);
  return NULL;
}

/* returns number of failing patterns in [start, end); first failure in *first */
int64_t walk(const double* val, const double* up, const double* down, void* rd, void* ru,
             uint64_t start, uint64_t end, int nthreads, uint32_t* first) {
  job_t jobs[64];
  pthread_t th[64];
  if (nthreads > 64) nthreads = 64;
  uint64_t span = (end - start + (uint64_t)nthreads - 1) / (uint64_t)nthreads;
  for (int t = 0; t < nthreads; t++) {
    jobs[t].val = val;
    jobs[t].up = up;
    jobs[t].down = down;
    jobs[t].rd = (round_fn)rd;
    jobs[t].ru = (round_fn)ru;
    jobs[t].start = start + span * (uint64_t)t;
    jobs[t].end = jobs[t].start + span < end ? jobs[t].start + span : end;
    if (jobs[t].start > end) jobs[t].start = end;
    jobs[t].fails = 0;
    jobs[t].first_fail = 0;
    pthread_create(&th[t], NULL, worker, &jobs[t]);
  }
  int64_t fails = 0;
  *first = 0;
  for (int t = 0; t < nthreads; t++) {
    pthread_join(th[t], NULL);
    if (jobs[t].fails && fails == 0) *first = jobs[t].first_fail;
    fails += jobs[t].fails;
  }
  return fails;
}
