/*
 * Seeded synthetic gradient values, host side.
 *
 * This file is input generation only: it holds none of the reduction's
 * arithmetic and is shared by the CPU oracle and by the GPU tests as the one
 * source of input values.  synth/gen_dev.hip implements the same generator
 * for the GPU; the two must agree byte for byte.
 *
 * Definition (integer operations only, so every implementation agrees):
 *   mix(z)      = SplitMix64 output function (Steele, Lea & Flood,
 *                 "Fast splittable pseudorandom number generators", OOPSLA
 *                 2014): z ^= z>>30; z *= 0xBF58476D1CE4E5B9; z ^= z>>27;
 *                 z *= 0x94D049BB133111EB; z ^= z>>31.
 *   G           = 0x9E3779B97F4A7C15 (the SplitMix64 increment).
 *   key(s, t)   = mix(mix(s + G) + (t + 1) G)        seed s, stream t
 *   h           = mix(key + (i + 1) G),  h2 = mix(h + G)   column i
 *   k           = sum of the four 16-bit fields of h, minus 131070
 *                 (Irwin-Hall of 4, integer, std 37837.23)
 *   m           = |k| * 2^24 + (h2 >> 40)            |k| plus a 24-bit fraction
 *   n           = m * C                              exact in 64 bits
 *   value       = (-1)^neg * n * 2^-(24+E), truncated to the format's
 *                 significand (24 bits fp32, 8 bits bf16); neg = k < 0,
 *                 or bit 0 of h2 when k == 0.
 * The value is approximately N(0, 37837.23 * C * 2^-E); C in [2^15, 2^16)
 * and E are chosen per workload.  With E <= 100 every value is a normal
 * number (or zero), so inputs never hold subnormals, infinities or NaNs.
 */
#include <stdint.h>
#include <stddef.h>

#define SYNTH_G 0x9E3779B97F4A7C15ULL

static inline uint64_t synth_mix(uint64_t z) {
  z ^= z >> 30;
  z *= 0xBF58476D1CE4E5B9ULL;
  z ^= z >> 27;
  z *= 0x94D049BB133111EBULL;
  z ^= z >> 31;
  return z;
}

uint64_t synth_key(uint64_t seed, uint64_t stream) {
  return synth_mix(synth_mix(seed + SYNTH_G) + (stream + 1) * SYNTH_G);
}

static inline uint32_t synth_bits(uint64_t key, uint64_t i, uint32_t C, uint32_t E, int bf16) {
  uint64_t h = synth_mix(key + (i + 1) * SYNTH_G);
  uint64_t h2 = synth_mix(h + SYNTH_G);
  int64_t k = (int64_t)(h & 0xFFFF) + (int64_t)((h >> 16) & 0xFFFF) +
              (int64_t)((h >> 32) & 0xFFFF) + (int64_t)(h >> 48) - 131070;
  uint32_t neg = (k < 0) || (k == 0 && (h2 & 1));
  uint64_t mag = (uint64_t)(k < 0 ? -k : k);
  uint64_t n = ((mag << 24) | (h2 >> 40)) * (uint64_t)C;
  if (n == 0) return bf16 ? (neg << 15) : (neg << 31);
  int L = 64 - __builtin_clzll(n);
  uint32_t bexp = (uint32_t)(L - 1 - 24 - (int)E + 127);
  if (bf16) {
    uint64_t sig = L > 8 ? n >> (L - 8) : n << (8 - L);
    return (neg << 15) | (bexp << 7) | (uint32_t)(sig & 0x7F);
  }
  uint64_t sig = L > 24 ? n >> (L - 24) : n << (24 - L);
  return (neg << 31) | (bexp << 23) | (uint32_t)(sig & 0x7FFFFF);
}

/* out[k] = value(seed, stream, column col0 + k) for k in [0, n).
 * dtype 0: bf16 (out is uint16_t*), dtype 1: fp32 (out is uint32_t*). */
void synth_fill_host(int dtype, uint64_t seed, uint64_t stream, uint32_t C, uint32_t E,
                     int64_t col0, int64_t n, void* out) {
  uint64_t key = synth_key(seed, stream);
  if (dtype == 0) {
    uint16_t* o = (uint16_t*)out;
#pragma omp parallel for schedule(static) if (n > 65536)
    for (int64_t k = 0; k < n; ++k) o[k] = (uint16_t)synth_bits(key, (uint64_t)(col0 + k), C, E, 1);
  } else {
    uint32_t* o = (uint32_t*)out;
#pragma omp parallel for schedule(static) if (n > 65536)
    for (int64_t k = 0; k < n; ++k) o[k] = synth_bits(key, (uint64_t)(col0 + k), C, E, 0);
  }
}

/* Gather form: out[k] = value(seed, stream, cols[k]); used to rebuild the
 * inputs of sampled columns of a full-size slab without materialising it. */
void synth_gather_host(int dtype, uint64_t seed, uint64_t stream, uint32_t C, uint32_t E,
                       const int64_t* cols, int64_t n, void* out) {
  uint64_t key = synth_key(seed, stream);
  if (dtype == 0) {
    uint16_t* o = (uint16_t*)out;
    for (int64_t k = 0; k < n; ++k) o[k] = (uint16_t)synth_bits(key, (uint64_t)cols[k], C, E, 1);
  } else {
    uint32_t* o = (uint32_t*)out;
    for (int64_t k = 0; k < n; ++k) o[k] = synth_bits(key, (uint64_t)cols[k], C, E, 0);
  }
}
