/*
 * synth_core.h - counter-based seeded generator for synthetic KDA inputs.
 *
 * This header is the single definition of every synthetic input value used by
 * the tests, the benchmark and the oracle checks.  It is compiled twice: by gcc
 * for the host filler (synth_host.c) and by hipcc for the device filler
 * (synth_dev.hip).  It contains no part of the KDA method; it only turns
 * (seed, tensor id, step, element index) into a number.
 *
 * Generator: SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014).  The n-th output of a SplitMix64 stream
 * whose state starts at `key` is mix64(key + (n + 1) * GAMMA); because that is
 * a pure function of n, any element can be regenerated without state, which is
 * what lets a 1M-token tensor be produced in slices or on the device.
 *
 * Normal deviates: Box-Muller (Box & Muller 1958), cosine branch only.  Element
 * e of a stream takes outputs 2e and 2e+1:
 *     u1 = ((x0 >> 11) + 1) * 2^-53    in (0, 1]
 *     u2 =  (x1 >> 11)      * 2^-53    in [0, 1)
 *     z  = sqrt(-2 ln u1) * cos(2 pi u2)
 *     x  = mean + std * z                      (fp64, no fused multiply-add)
 * then rounded fp64 -> fp32 (round-to-nearest-even) and, for bf16 tensors,
 * fp32 -> bf16 (round-to-nearest-even).
 *
 * The includer defines SYNTH_FN (the function qualifiers) before including.
 */
#ifndef SYNTH_CORE_H
#define SYNTH_CORE_H

#include <stdint.h>

#ifndef SYNTH_FN
#error "define SYNTH_FN before including synth_core.h"
#endif

#define SYNTH_GAMMA 0x9E3779B97F4A7C15ULL
#define SYNTH_TWO_PI 6.283185307179586 /* nearest double to 2*pi */
#define SYNTH_TWO_M53 1.1102230246251565e-16 /* 2^-53, exact */

/* SplitMix64 output function (the "mix" applied to the advanced state). */
SYNTH_FN uint64_t synth_mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* Stream key for one tensor of one workload: distinct (seed, tensor, step)
 * triples give unrelated streams. */
SYNTH_FN uint64_t synth_stream_key(uint64_t seed, uint32_t tensor, uint32_t step) {
  uint64_t tag = ((uint64_t)tensor << 32) | (uint64_t)step;
  return synth_mix64(synth_mix64(seed + SYNTH_GAMMA) ^ synth_mix64(tag + 2 * SYNTH_GAMMA));
}

/* n-th raw 64-bit output of the stream. */
SYNTH_FN uint64_t synth_u64(uint64_t key, uint64_t n) {
  return synth_mix64(key + (n + 1) * SYNTH_GAMMA);
}

/* 53-bit uniform in [0, 1). */
SYNTH_FN double synth_uniform(uint64_t key, uint64_t n) {
  return (double)(synth_u64(key, n) >> 11) * SYNTH_TWO_M53;
}

/* Normal deviate for element e (Box-Muller, cosine branch), in fp64.
 * sqrt/log/cos come from the includer's math library (libm on the host, the
 * ROCm device library on the GPU); the includer must compile with
 * floating-point contraction off so mean + std * z is not fused. */
SYNTH_FN double synth_normal(uint64_t key, uint64_t e, double mean, double std) {
  double u1 = (double)((synth_u64(key, 2 * e) >> 11) + 1) * SYNTH_TWO_M53;
  double u2 = (double)(synth_u64(key, 2 * e + 1) >> 11) * SYNTH_TWO_M53;
  double r = sqrt(-2.0 * log(u1));
  double z = r * cos(SYNTH_TWO_PI * u2);
  double s = std * z;
  return mean + s;
}

/* fp32 -> bf16 bits, round to nearest even (inputs are finite). */
SYNTH_FN uint16_t synth_f32_to_bf16(float f) {
  union { float f; uint32_t u; } c;
  c.f = f;
  uint32_t u = c.u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

#endif /* SYNTH_CORE_H */
