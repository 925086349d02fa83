/* Exhaustive pin of the oracle's fp32 -> bf16 rounding: every one of the 2^32
 * fp32 bit patterns against a rounder written from the definition (the nearer
 * of the two bf16 neighbours by exact distance, ties to the even pattern, the
 * upper neighbour taken with an unbounded exponent so that values at or above
 * max + half an ulp go to infinity; NaN -> quiet NaN 0x7FC0 with its sign).
 * Distances are exact in double: both neighbours share the value's exponent
 * range and carry at most 24 significant bits.  Test infrastructure: it links
 * the oracle library and shares no code with it. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

uint16_t or_f32_to_bf16(float f);

static double val16(uint32_t p) {
  uint32_t e = p >> 7, m = p & 0x7F;
  if (e == 0) return ldexp((double)m, -133);
  return ldexp((double)(m + 128), (int)e - 134);
}

static uint16_t def_round(uint32_t u) {
  uint32_t sign = u >> 31, mag = u & 0x7FFFFFFFu;
  if (mag > 0x7F800000u) return (uint16_t)((sign << 15) | 0x7FC0u);
  if (mag == 0x7F800000u) return (uint16_t)((sign << 15) | 0x7F80u);
  uint32_t e = mag >> 23, m = mag & 0x7FFFFFu;
  double f = e == 0 ? ldexp((double)m, -149) : ldexp((double)(m | 0x800000u), (int)e - 150);
  uint32_t lo = mag >> 16, hi = lo + 1;
  double dlo = f - val16(lo), dhi = val16(hi) - f;
  uint32_t pick = (dhi < dlo || (dhi == dlo && (lo & 1u))) ? hi : lo;
  return (uint16_t)((sign << 15) | pick);
}

int main(void) {
  long long bad = 0;
  uint32_t first = 0;
#pragma omp parallel for reduction(+ : bad) schedule(static)
  for (long long i = 0; i < (1LL << 32); ++i) {
    uint32_t u = (uint32_t)i;
    float f;
    memcpy(&f, &u, 4);
    if (or_f32_to_bf16(f) != def_round(u)) {
      if (bad == 0) first = u;
      ++bad;
    }
  }
  printf("%lld mismatches over 2^32 patterns (first 0x%08x)\n", bad, first);
  return bad != 0;
}
