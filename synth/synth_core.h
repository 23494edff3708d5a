/*
 * synth_core.h -- seeded synthetic input generator shared by the CPU oracle
 * side and the GPU side.  It holds no arithmetic of the quantized MoE method:
 * only a counter-based integer hash, an integer sum that approximates a normal
 * draw, and fp32 -> bf16 rounding of the drawn values (an input format).
 *
 * The same source is compiled by gcc (host) and by hipcc (device), so every
 * value is a pure function of (seed, stream, element index) and is
 * bit-identical on both: all steps are integer operations, followed by
 * exactly-representable conversions and one correctly rounded fp32 multiply.
 *
 * Generator: SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014): state_i = base + (i+1)*gamma, output =
 * mix64(state_i) with the variant-13 finaliser used by SplittableRandom.
 *
 * Normal approximation: Irwin-Hall with 12 uniforms -- the sum of twelve
 * 16-bit uniforms minus its mean, scaled by 2^-16.  Mean 0, variance
 * 1 - 2^-32, support [-6, 6].  Every intermediate is an integer below 2^20,
 * so the fp32 value is exact on any IEEE machine.
 */
#ifndef SYNTH_CORE_H
#define SYNTH_CORE_H

#include <stdint.h>

#if defined(__HIPCC__)
#define SYNTH_FN __host__ __device__ static inline
#else
#define SYNTH_FN static inline
#endif

#define SYNTH_GAMMA 0x9E3779B97F4A7C15ull

/* Stream tags: one independent stream per generated tensor. */
enum {
  SYNTH_STREAM_X = 1,        /* activations */
  SYNTH_STREAM_X_OUTLIER = 2,/* outlier mask of the activations */
  SYNTH_STREAM_LOGITS = 3,   /* gate logits */
  SYNTH_STREAM_W13 = 4,      /* gate+up expert weights */
  SYNTH_STREAM_W2 = 5,       /* down expert weights */
  SYNTH_STREAM_PERM = 6,     /* expert popularity permutation */
  SYNTH_STREAM_MISC = 7      /* anything else a test draws */
};

SYNTH_FN uint64_t synth_mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

/* Base state of one (seed, stream) pair. */
SYNTH_FN uint64_t synth_base(uint64_t seed, uint64_t stream) {
  return synth_mix64(synth_mix64(seed * SYNTH_GAMMA + 0x632BE59BD9B4E019ull) ^ (stream * 0xD1B54A32D192ED03ull));
}

/* j-th 64-bit output of the stream. */
SYNTH_FN uint64_t synth_u64(uint64_t base, uint64_t j) {
  return synth_mix64(base + (j + 1ull) * SYNTH_GAMMA);
}

/* Sum of the four 16-bit fields of a 64-bit word. */
SYNTH_FN uint32_t synth_sum16x4(uint64_t v) {
  return (uint32_t)(v & 0xFFFFull) + (uint32_t)((v >> 16) & 0xFFFFull) +
         (uint32_t)((v >> 32) & 0xFFFFull) + (uint32_t)(v >> 48);
}

/* Approximate standard normal for element i: uses words 3i, 3i+1, 3i+2. */
SYNTH_FN float synth_normal(uint64_t base, uint64_t i) {
  uint32_t s = synth_sum16x4(synth_u64(base, 3ull * i)) +
               synth_sum16x4(synth_u64(base, 3ull * i + 1ull)) +
               synth_sum16x4(synth_u64(base, 3ull * i + 2ull));
  int32_t c = (int32_t)s - 393210; /* 12 * 32767.5 */
  return (float)c * (1.0f / 65536.0f);
}

/* Uniform 32-bit integer for element i. */
SYNTH_FN uint32_t synth_u32(uint64_t base, uint64_t i) {
  return (uint32_t)(synth_u64(base, i) >> 32);
}

/* fp32 -> bf16 bits, round to nearest even (inputs here are always finite). */
SYNTH_FN uint16_t synth_f32_to_bf16(float f) {
  union { float f; uint32_t u; } v;
  v.f = f;
  uint32_t rounding = 0x7FFFu + ((v.u >> 16) & 1u);
  return (uint16_t)((v.u + rounding) >> 16);
}

/* Outlier probability 1% as a threshold on a 32-bit uniform: floor(0.01 * 2^32). */
#define SYNTH_OUTLIER_THRESHOLD 42949672u

/* Activation element i: sigma * z, multiplied by `mult` when the element is an outlier. */
SYNTH_FN float synth_activation(uint64_t base_x, uint64_t base_o, uint64_t i, float sigma,
                                uint32_t outlier_threshold, float mult) {
  float v = synth_normal(base_x, i) * sigma;
  if (synth_u32(base_o, i) < outlier_threshold) v = v * mult;
  return v;
}

#endif /* SYNTH_CORE_H */
