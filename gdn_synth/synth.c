/*
 * Seeded synthetic numbers for the GDN prefill workloads (no arithmetic of the
 * method itself lives here).
 *
 * SplitMix64 (Steele, Lea and Flood, OOPSLA 2014) in counter form: value i of the
 * stream with seed s is mix(s + (i + 1) * 0x9E3779B97F4A7C15), where mix is the
 * SplitMix64 finaliser. A tensor's stream seed is mix(seed ^ tensor_id).
 * Uniforms: (z >> 11) * 2^-53. Normals: Box-Muller (1958) on the uniform pair
 * (2p, 2p + 1): r = sqrt(-2 log(1 - u1)), theta = 2 pi u2, element 2p = r cos theta,
 * element 2p + 1 = r sin theta, all in fp64. A drawn value is x * std + mean in
 * fp64, rounded to fp32 (nearest even), and for bf16 tensors then to bf16
 * (nearest even).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

static uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

uint64_t synth_stream_seed(uint64_t seed, uint64_t tensor_id) { return mix64(seed ^ tensor_id); }

static double uni(uint64_t sseed, uint64_t i) {
  const uint64_t z = mix64(sseed + (i + 1) * 0x9E3779B97F4A7C15ULL);
  return (double)(z >> 11) * (1.0 / 9007199254740992.0);
}

void synth_uniform(uint64_t seed, uint64_t tensor_id, int64_t start, int64_t n, double* out) {
  const uint64_t s = synth_stream_seed(seed, tensor_id);
  for (int64_t i = 0; i < n; ++i) out[i] = uni(s, (uint64_t)(start + i));
}

static double normal_at(uint64_t sseed, int64_t i) {
  const int64_t p = i >> 1;
  const double u1 = uni(sseed, (uint64_t)(2 * p)), u2 = uni(sseed, (uint64_t)(2 * p + 1));
  const double r = sqrt(-2.0 * log1p(-u1));
  const double th = 6.283185307179586 * u2;
  return (i & 1) ? r * sin(th) : r * cos(th);
}

static uint16_t f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += ((u >> 16) & 1u) + 0x7FFFu;
  return (uint16_t)(u >> 16);
}

typedef struct {
  uint64_t sseed;
  int64_t lo, hi;
  double mean, std;
  int bf16;
  void* out;
} job_t;

static void* run(void* arg) {
  job_t* J = (job_t*)arg;
  for (int64_t i = J->lo; i < J->hi; ++i) {
    const float f = (float)(normal_at(J->sseed, i) * J->std + J->mean);
    if (J->bf16)
      ((uint16_t*)J->out)[i] = f32_to_bf16(f);
    else
      ((float*)J->out)[i] = f;
  }
  return NULL;
}

/* n normals * std + mean into out (float32 if bf16 == 0, else bf16 bit patterns). */
void synth_normal(uint64_t seed, uint64_t tensor_id, int64_t n, double mean, double std,
                  int bf16, void* out, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 64) nthreads = 64;
  if (n < 65536) nthreads = 1;
  job_t jobs[64];
  pthread_t th[64];
  const uint64_t s = synth_stream_seed(seed, tensor_id);
  for (int t = 0; t < nthreads; ++t) {
    jobs[t].sseed = s;
    jobs[t].lo = n * t / nthreads;
    jobs[t].hi = n * (t + 1) / nthreads;
    jobs[t].mean = mean;
    jobs[t].std = std;
    jobs[t].bf16 = bf16;
    jobs[t].out = out;
  }
  for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, run, &jobs[t]);
  run(&jobs[0]);
  for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
}

/* n normals * std + mean in fp64 (no rounding). */
void synth_normal_f64(uint64_t seed, uint64_t tensor_id, int64_t n, double mean, double std,
                      double* out) {
  const uint64_t s = synth_stream_seed(seed, tensor_id);
  for (int64_t i = 0; i < n; ++i) out[i] = normal_at(s, i) * std + mean;
}
