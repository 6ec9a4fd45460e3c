/*
 * Seeded synthetic input generator (host C, OpenMP).
 *
 * This file holds no arithmetic of the method under test: it only turns
 * (seed, stream, index) identities into Gaussian values and stores them in the
 * element type the workload uses.  Both the GPU library's tests and the CPU
 * oracle consume the arrays it writes; neither side links against this file.
 *
 * Random numbers: SplitMix64 (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014) used as a counter-based
 * generator.  The key of stream s under seed S is the s-th output of a
 * SplitMix64 sequence started at state S; value c of that stream is the c-th
 * output of a sequence started at the key.  Uniforms take the top 53 bits,
 * offset by one half ulp so they lie strictly inside (0, 1).  Normals use the
 * Box-Muller transform: identity i uses uniform pair (2*(i/2), 2*(i/2)+1) and
 * takes the cosine branch for even i, the sine branch for odd i.
 *
 * Storage rounding: fp64 -> fp32 by the C cast (round to nearest even), then
 * fp32 -> bf16 by round to nearest even on the bit pattern.  (Two roundings; the
 * stored values are the inputs both sides see, so this only shapes the input
 * distribution.)
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* c-th output (c >= 0) of a SplitMix64 sequence whose state starts at s. */
static inline uint64_t sm_at(uint64_t s, uint64_t c) { return mix64(s + (c + 1) * GAMMA); }

uint64_t synth_stream_key(uint64_t seed, uint64_t stream) { return sm_at(seed, stream); }

static inline double unif(uint64_t key, uint64_t c) {
  return ((double)(sm_at(key, c) >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}

static inline double normal_at(uint64_t key, uint64_t id) {
  const uint64_t j = id >> 1;
  const double u1 = unif(key, 2 * j), u2 = unif(key, 2 * j + 1);
  const double r = sqrt(-2.0 * log(u1));
  const double a = 6.283185307179586476925287 * u2;
  return (id & 1) ? r * sin(a) : r * cos(a);
}

static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* Store v at out[i] in element type kind: 0 = fp64, 1 = fp32, 2 = bf16 bits. */
static inline void store(void* out, int64_t i, int kind, double v) {
  if (kind == 0) ((double*)out)[i] = v;
  else if (kind == 1) ((float*)out)[i] = (float)v;
  else ((uint16_t*)out)[i] = f32_to_bf16_rne((float)v);
}

/* Standard normals of one stream, identities [start, start+n), fp64 out. */
void synth_normals(uint64_t seed, uint64_t stream, int64_t start, int64_t n, double* out) {
  const uint64_t key = synth_stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = normal_at(key, (uint64_t)(start + i));
}

/* Uniforms in (0, 1) of one stream, identities [start, start+n), rounded to fp32 (which can
 * reach 1.0f for the very largest draws). */
void synth_uniforms_f32(uint64_t seed, uint64_t stream, int64_t start, int64_t n, float* out) {
  const uint64_t key = synth_stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = (float)unif(key, (uint64_t)(start + i));
}

/*
 * Dense rows: out[r*cols + c] = scale * N(stream, src_row[r]*cols + c)
 *                               * (row_sigma != 0 ? exp(row_sigma * N(row_stream, src_row[r])) : 1)
 * src_row == NULL means src_row[r] = r + row0.  Rows that share a source row
 * receive identical values (used to plant exact duplicates).
 */
void synth_rows(uint64_t seed, uint64_t stream, const int64_t* src_row, int64_t row0,
                int64_t rows, int64_t cols, double scale, double row_sigma,
                uint64_t row_stream, int kind, void* out) {
  const uint64_t key = synth_stream_key(seed, stream);
  const uint64_t rkey = synth_stream_key(seed, row_stream);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    const int64_t s = src_row ? src_row[r] : r + row0;
    double f = scale;
    if (row_sigma != 0.0) f *= exp(row_sigma * normal_at(rkey, (uint64_t)s));
    for (int64_t c = 0; c < cols; ++c)
      store(out, r * cols + c, kind, f * normal_at(key, (uint64_t)(s * cols + c)));
  }
}

/*
 * Saved SwiGLU activations: row r is the activation of source pair src[r]:
 *   a, c ~ N(0,1) (streams sa, sc, identity src*cols + j);  v = a / (1 + exp(-a)) * c,
 * optionally times exp(row_sigma * N(row_stream, src)).
 */
void synth_swiglu_rows(uint64_t seed, uint64_t sa, uint64_t sc, const int64_t* src, int64_t rows,
                       int64_t cols, double row_sigma, uint64_t row_stream, int kind, void* out) {
  const uint64_t ka = synth_stream_key(seed, sa), kc = synth_stream_key(seed, sc);
  const uint64_t rkey = synth_stream_key(seed, row_stream);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    const int64_t s = src[r];
    double f = 1.0;
    if (row_sigma != 0.0) f = exp(row_sigma * normal_at(rkey, (uint64_t)s));
    for (int64_t j = 0; j < cols; ++j) {
      const uint64_t id = (uint64_t)(s * cols + j);
      const double a = normal_at(ka, id), c = normal_at(kc, id);
      store(out, r * cols + j, kind, f * (a / (1.0 + exp(-a))) * c);
    }
  }
}

/*
 * Saved FC1 outputs of the same pairs: row r holds the gate pre-activation a in columns [0, cols)
 * and the up projection f*c in columns [cols, 2*cols), where a, c and the row scale f are the very
 * draws synth_swiglu_rows turns into SiLU(a)*c*f.
 */
void synth_swiglu_context(uint64_t seed, uint64_t sa, uint64_t sc, const int64_t* src,
                          int64_t rows, int64_t cols, double row_sigma, uint64_t row_stream,
                          int kind, void* out) {
  const uint64_t ka = synth_stream_key(seed, sa), kc = synth_stream_key(seed, sc);
  const uint64_t rkey = synth_stream_key(seed, row_stream);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    const int64_t s = src[r];
    double f = 1.0;
    if (row_sigma != 0.0) f = exp(row_sigma * normal_at(rkey, (uint64_t)s));
    for (int64_t j = 0; j < cols; ++j) {
      const uint64_t id = (uint64_t)(s * cols + j);
      store(out, r * 2 * cols + j, kind, normal_at(ka, id));
      store(out, r * 2 * cols + cols + j, kind, f * normal_at(kc, id));
    }
  }
}
