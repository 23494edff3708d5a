/*
 * synth_host.c -- host (CPU) fills of the seeded synthetic inputs.
 * Every element is a pure function of (seed, stream, index) defined in
 * synth_core.h; the device fills in synth_dev.hip produce identical bits.
 */
#include "synth_core.h"

#include <stddef.h>

#define SYNTH_EXPORT __attribute__((visibility("default")))

/* out[i] = sigma * N(0,1) draw number (start + i) of the stream. */
SYNTH_EXPORT void synth_fill_normal_f32(float* out, int64_t n, uint64_t seed, uint64_t stream,
                                        int64_t start, float sigma) {
  const uint64_t base = synth_base(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = synth_normal(base, (uint64_t)(start + i)) * sigma;
}

/* Gate logits: out[t,e] = z[(row_start+t)*E + e] + bias[e] (bias may be NULL). */
SYNTH_EXPORT void synth_fill_logits_f32(float* out, int64_t T, int64_t E, uint64_t seed,
                                        const float* bias, int64_t row_start) {
  const uint64_t base = synth_base(seed, SYNTH_STREAM_LOGITS);
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t e = 0; e < E; ++e) {
      float z = synth_normal(base, (uint64_t)((row_start + t) * E + e));
      out[t * E + e] = bias ? z + bias[e] : z;
    }
  }
}

/* Activations [rows, cols]: sigma * z, times `mult` on the outlier mask.
   dtype 0 writes fp32, dtype 1 writes bf16 bits (round to nearest even). */
SYNTH_EXPORT void synth_fill_activation(void* out, int32_t dtype, int64_t rows, int64_t cols,
                                        uint64_t seed, float sigma, uint32_t outlier_threshold,
                                        float mult, int64_t row_start) {
  const uint64_t bx = synth_base(seed, SYNTH_STREAM_X);
  const uint64_t bo = synth_base(seed, SYNTH_STREAM_X_OUTLIER);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t c = 0; c < cols; ++c) {
      uint64_t i = (uint64_t)((row_start + r) * cols + c);
      float v = synth_activation(bx, bo, i, sigma, outlier_threshold, mult);
      if (dtype == 1)
        ((uint16_t*)out)[r * cols + c] = synth_f32_to_bf16(v);
      else
        ((float*)out)[r * cols + c] = v;
    }
  }
}

/* Seeded Fisher-Yates permutation of 0..n-1 (draw j picks from [0, i]). */
SYNTH_EXPORT void synth_permutation(int32_t* perm, int64_t n, uint64_t seed) {
  const uint64_t base = synth_base(seed, SYNTH_STREAM_PERM);
  for (int64_t i = 0; i < n; ++i) perm[i] = (int32_t)i;
  for (int64_t i = n - 1; i > 0; --i) {
    uint64_t r = synth_u64(base, (uint64_t)i) % (uint64_t)(i + 1);
    int32_t tmp = perm[i];
    perm[i] = perm[r];
    perm[r] = tmp;
  }
}

/* Raw 64-bit words of a stream, for the generator's own tests. */
SYNTH_EXPORT void synth_words(uint64_t* out, int64_t n, uint64_t seed, uint64_t stream, int64_t start) {
  const uint64_t base = synth_base(seed, stream);
  for (int64_t i = 0; i < n; ++i) out[i] = synth_u64(base, (uint64_t)(start + i));
}

/* Plain SplitMix64 sequence from a raw state (state += gamma; output mix64(state)),
   for checking the generator against its published reference outputs. */
SYNTH_EXPORT void synth_splitmix64(uint64_t* out, int64_t n, uint64_t state) {
  for (int64_t i = 0; i < n; ++i) out[i] = synth_u64(state, (uint64_t)i);
}
