/*
 * Seeded synthetic tensors for the MoE feed-forward workloads.
 *
 * This file makes input DATA only: it holds none of the layer's arithmetic
 * (no routing, no expert math). Both the CPU oracle and the GPU path take
 * their inputs from here, so the two sides always see the same bits.
 *
 * Generator: Philox-4x32-10, the counter-based generator of Salmon, Moraes,
 * Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3" (SC'11).
 * Each 128-bit counter is encrypted by ten rounds of a multiply/xor bijection
 * with a 64-bit key that is bumped by a Weyl sequence after every round.
 *
 *   counter = (j_lo, j_hi, tensor_id, stream), key = (seed_lo, seed_hi)
 *
 * Normal values: element pair (2j, 2j+1) comes from counter j via the
 * Box-Muller transform in double precision, then is multiplied by `scale`
 * and rounded to float (round-to-nearest-even); bf16 tensors are rounded
 * once more from that float to bf16 (round-to-nearest-even).
 * Uniform int8 values: element i takes word (i mod 4) of counter i/4 and maps
 * the 32-bit word w to floor(w * 255 / 2^32) - 127, an integer in [-127, 127].
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

static inline void mulhilo32(uint32_t a, uint32_t b, uint32_t* hi, uint32_t* lo) {
  uint64_t p = (uint64_t)a * (uint64_t)b;
  *hi = (uint32_t)(p >> 32);
  *lo = (uint32_t)p;
}

void syn_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
  uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
  uint32_t k0 = key_in[0], k1 = key_in[1];
  for (int r = 0; r < 10; ++r) {
    uint32_t hi0, lo0, hi1, lo1;
    mulhilo32(PHILOX_M0, c0, &hi0, &lo0);
    mulhilo32(PHILOX_M1, c2, &hi1, &lo1);
    uint32_t n0 = hi1 ^ c1 ^ k0;
    uint32_t n1 = lo1;
    uint32_t n2 = hi0 ^ c3 ^ k1;
    uint32_t n3 = lo0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    k0 += PHILOX_W0;
    k1 += PHILOX_W1;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* Two standard normals from one counter (Box-Muller, double precision). */
static inline void normal_pair(uint64_t j, uint32_t tensor_id, uint64_t seed, double* z0, double* z1) {
  uint32_t ctr[4] = {(uint32_t)j, (uint32_t)(j >> 32), tensor_id, 0u};
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t w[4];
  syn_philox4x32_10(ctr, key, w);
  uint64_t a = ((uint64_t)w[0] << 21) | (w[1] >> 11); /* 53 bits */
  uint64_t b = ((uint64_t)w[2] << 21) | (w[3] >> 11);
  double u1 = ((double)a + 1.0) * 0x1.0p-53; /* (0, 1] */
  double u2 = (double)b * 0x1.0p-53;         /* [0, 1) */
  double r = sqrt(-2.0 * log(u1));
  double t = 6.283185307179586476925286766559 * u2;
  *z0 = r * cos(t);
  *z1 = r * sin(t);
}

enum { KIND_F32 = 0, KIND_BF16 = 1, KIND_I8 = 2 };

typedef struct {
  void* out;
  int kind;
  int64_t begin, end; /* element range, begin even */
  uint64_t seed;
  uint32_t tensor_id;
  double scale;
} job_t;

static void* run_job(void* p) {
  job_t* jb = (job_t*)p;
  if (jb->kind == KIND_I8) {
    int8_t* o = (int8_t*)jb->out;
    uint32_t key[2] = {(uint32_t)jb->seed, (uint32_t)(jb->seed >> 32)};
    for (int64_t i = jb->begin; i < jb->end;) {
      uint64_t j = (uint64_t)i >> 2;
      uint32_t ctr[4] = {(uint32_t)j, (uint32_t)(j >> 32), jb->tensor_id, 1u};
      uint32_t w[4];
      syn_philox4x32_10(ctr, key, w);
      for (int s = (int)(i & 3); s < 4 && i < jb->end; ++s, ++i)
        o[i] = (int8_t)((int)(((uint64_t)w[s] * 255u) >> 32) - 127);
    }
    return 0;
  }
  for (int64_t i = jb->begin; i < jb->end; i += 2) {
    double z0, z1;
    normal_pair((uint64_t)i >> 1, jb->tensor_id, jb->seed, &z0, &z1);
    float v0 = (float)(z0 * jb->scale), v1 = (float)(z1 * jb->scale);
    if (jb->kind == KIND_F32) {
      float* o = (float*)jb->out;
      o[i] = v0;
      if (i + 1 < jb->end) o[i + 1] = v1;
    } else {
      uint16_t* o = (uint16_t*)jb->out;
      o[i] = f32_to_bf16_rne(v0);
      if (i + 1 < jb->end) o[i + 1] = f32_to_bf16_rne(v1);
    }
  }
  return 0;
}

static void run_parallel(void* out, int kind, int64_t n, uint64_t seed, uint32_t tensor_id,
                         double scale, int nthreads) {
  if (n <= 0) return;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  int64_t per = (n + nthreads - 1) / nthreads;
  per = (per + 7) & ~(int64_t)7; /* keep chunk starts aligned to pairs and quads */
  pthread_t th[256];
  job_t jobs[256];
  int started = 0;
  for (int t = 0; t < nthreads; ++t) {
    int64_t b = (int64_t)t * per, e = b + per;
    if (b >= n) break;
    if (e > n) e = n;
    jobs[t] = (job_t){out, kind, b, e, seed, tensor_id, scale};
    if (nthreads == 1 || pthread_create(&th[t], 0, run_job, &jobs[t]) != 0) {
      run_job(&jobs[t]);
      th[t] = 0;
    }
    started = t + 1;
  }
  for (int t = 0; t < started; ++t)
    if (th[t]) pthread_join(th[t], 0);
}

/* n normals times `scale`, as float. */
void syn_normal_f32(float* out, int64_t n, uint64_t seed, uint32_t tensor_id, double scale, int nthreads) {
  run_parallel(out, KIND_F32, n, seed, tensor_id, scale, nthreads);
}

/* n normals times `scale`, rounded to float then to bf16 (bit patterns). */
void syn_normal_bf16(uint16_t* out, int64_t n, uint64_t seed, uint32_t tensor_id, double scale, int nthreads) {
  run_parallel(out, KIND_BF16, n, seed, tensor_id, scale, nthreads);
}

/* n integers uniform in [-127, 127]. */
void syn_uniform_i8(int8_t* out, int64_t n, uint64_t seed, uint32_t tensor_id, int nthreads) {
  run_parallel(out, KIND_I8, n, seed, tensor_id, 0.0, nthreads);
}
