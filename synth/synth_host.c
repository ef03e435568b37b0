/*
 * synth_host.c - host (CPU) filler for the seeded synthetic inputs.
 * Built with gcc -ffp-contract=off; see synth_core.h for the value definition.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define SYNTH_FN static inline
#include "synth_core.h"

enum { SYNTH_F32 = 0, SYNTH_BF16 = 1 };

uint64_t synth_key(uint64_t seed, uint32_t tensor, uint32_t step) {
  return synth_stream_key(seed, tensor, step);
}

typedef struct {
  void* out;
  int dtype;
  uint64_t key;
  double mean, std;
  int64_t row_len, row_stride, base;
  int64_t r0, r1;
} fill_job;

static void* fill_rows(void* p) {
  fill_job* j = (fill_job*)p;
  for (int64_t r = j->r0; r < j->r1; ++r) {
    int64_t e0 = j->base + r * j->row_stride;
    for (int64_t c = 0; c < j->row_len; ++c) {
      double x = synth_normal(j->key, (uint64_t)(e0 + c), j->mean, j->std);
      float f = (float)x;
      int64_t o = r * j->row_len + c;
      if (j->dtype == SYNTH_F32)
        ((float*)j->out)[o] = f;
      else
        ((uint16_t*)j->out)[o] = synth_f32_to_bf16(f);
    }
  }
  return NULL;
}

/* out[r][c] (dense, n_rows x row_len) = value of element base + r*row_stride + c.
 * Returns 0 on success, -1 on a bad argument. */
int synth_fill_normal(void* out, int dtype, uint64_t key, double mean, double std,
                      int64_t n_rows, int64_t row_len, int64_t row_stride, int64_t base,
                      int nthreads) {
  if (!out || n_rows < 0 || row_len < 0 || base < 0 || (dtype != SYNTH_F32 && dtype != SYNTH_BF16))
    return -1;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (n_rows < nthreads) nthreads = n_rows > 0 ? (int)n_rows : 1;
  fill_job jobs[256];
  pthread_t th[256];
  int64_t per = (n_rows + nthreads - 1) / nthreads;
  for (int t = 0; t < nthreads; ++t) {
    jobs[t] = (fill_job){out, dtype, key, mean, std, row_len, row_stride, base, 0, 0};
    jobs[t].r0 = (int64_t)t * per < n_rows ? (int64_t)t * per : n_rows;
    jobs[t].r1 = jobs[t].r0 + per < n_rows ? jobs[t].r0 + per : n_rows;
  }
  for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, fill_rows, &jobs[t]);
  fill_rows(&jobs[0]);
  for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
  return 0;
}

/* n integers uniform on [lo, hi] inclusive: lo + floor(u * (hi - lo + 1)). */
int synth_uniform_ints(int32_t* out, int32_t n, uint64_t key, int32_t lo, int32_t hi) {
  if (!out || n < 0 || hi < lo) return -1;
  double span = (double)hi - (double)lo + 1.0;
  for (int32_t i = 0; i < n; ++i) {
    int64_t v = lo + (int64_t)(synth_uniform(key, (uint64_t)i) * span);
    out[i] = (int32_t)(v > hi ? hi : v);
  }
  return 0;
}
