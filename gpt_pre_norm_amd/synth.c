/* Native fill routines for the seeded synthetic-input generator.
 *
 * Same definition as the Python module next to it (gpt_pre_norm_amd/synth.py):
 * SplitMix64 words keyed by (seed, stream), Box-Muller normals, multiply-shift
 * token ids.  It holds none of the decoder's arithmetic.  Threads split the
 * index range; every element depends only on its own index, so the output does
 * not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>

static uint64_t mix64(uint64_t z) {
  z ^= z >> 30;
  z *= 0xBF58476D1CE4E5B9ULL;
  z ^= z >> 27;
  z *= 0x94D049BB133111EBULL;
  z ^= z >> 31;
  return z;
}

uint64_t synth_stream_key(uint64_t seed, uint64_t stream) {
  return mix64(mix64(seed) ^ (stream * 0xD1B54A32D192ED03ULL));
}

static inline uint64_t word_at(uint64_t key, uint64_t i) {
  return mix64(key + (i + 1) * 0x9E3779B97F4A7C15ULL);
}

static inline double uniform_at(uint64_t key, uint64_t i) {
  return ((double)(word_at(key, i) >> 11) + 0.5) * 0x1p-53;
}

static inline uint16_t f32_to_bf16_rne(float f) {
  union { float f; uint32_t u; } v = {f};
  uint32_t u = v.u;
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

static inline float bf16_to_f32(uint16_t b) {
  union { uint32_t u; float f; } v = {(uint32_t)b << 16};
  return v.f;
}

/* Both draws of Box-Muller pair p (elements 2p and 2p+1). */
static inline void normal_pair(uint64_t key, uint64_t p, double *z0, double *z1) {
  double u1 = uniform_at(key, 2 * p), u2 = uniform_at(key, 2 * p + 1);
  double r = sqrt(-2.0 * log(u1));
  double t = 2.0 * 3.14159265358979323846 * u2;
  *z0 = r * cos(t);
  *z1 = r * sin(t);
}

/* Calls put(i, z) for i in [0, count), z = N(0,1) draw of element start+i. */
#define FILL_NORMALS(PUT)                                                        \
  do {                                                                         \
    uint64_t p_lo = start >> 1, p_hi = (start + count + 1) >> 1;                \
    _Pragma("omp parallel for schedule(static)")                               \
    for (int64_t p = (int64_t)p_lo; p < (int64_t)p_hi; ++p) {                  \
      double z[2];                                                             \
      normal_pair(key, (uint64_t)p, &z[0], &z[1]);                             \
      for (int j = 0; j < 2; ++j) {                                            \
        uint64_t e = 2 * (uint64_t)p + j;                                      \
        if (e >= start && e < start + count) { PUT(e - start, z[j]); }         \
      }                                                                        \
    }                                                                          \
  } while (0)

/* out[i] = fp32(std * N(0,1) of element start+i); bf16-rounded when round_bf16 != 0 */
void synth_normal_f32(uint64_t seed, uint64_t stream, uint64_t start, uint64_t count,
                      double std, int round_bf16, float *out) {
  uint64_t key = synth_stream_key(seed, stream);
#define PUT_F32(i, z)                                                  \
  {                                                                    \
    float f = (float)((z) * std);                                      \
    out[i] = round_bf16 ? bf16_to_f32(f32_to_bf16_rne(f)) : f;         \
  }
  FILL_NORMALS(PUT_F32);
}

/* same draws, written as bf16 bit patterns */
void synth_normal_bf16(uint64_t seed, uint64_t stream, uint64_t start, uint64_t count,
                       double std, uint16_t *out) {
  uint64_t key = synth_stream_key(seed, stream);
#define PUT_BF16(i, z) { out[i] = f32_to_bf16_rne((float)((z) * std)); }
  FILL_NORMALS(PUT_BF16);
}

void synth_token_ids(uint64_t seed, uint64_t stream, uint64_t count, uint32_t n_vocab,
                     int32_t *out) {
  uint64_t key = synth_stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)count; ++i)
    out[i] = (int32_t)(((word_at(key, (uint64_t)i) >> 32) * (uint64_t)n_vocab) >> 32);
}
