// Host-side NF4 table for the HIP library.
//
// "QLoRA: Quantize Base Weights to 4-Bit", Section 2 "1. 4-bit NormalFloat": the 16 levels
// are q_i = (Q(i/17) + Q((i+1)/17)) / 2 with Q the standard-normal quantile (k = 4,
// 2^k + 1 = 17), so 0 is exact and the top level is finite.  "QLoRA -- Fine-Tuning a 65B
// Model on One GPU", "NF4": 8 negative levels, 8 non-negative ones including 0, and the
// endpoints pinned at exactly -1 and +1.
//
// Reading taken where the printed formula breaks down (i = 0 gives Q(0) = -inf): the tail
// level takes the quantile at its bin's probability midpoint, Q(1/34); each side is then
// divided by its own extreme (negatives by |q_0|, the rest by q_15).
//
// The quantile is computed here by bisection of Phi(x) = erfc(-x / sqrt 2) / 2 in x87
// long double; the result is rounded once to FP32.
#include <cfloat>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "qlora_host.h"

namespace qlora {
namespace {

long double phi(long double x) { return 0.5L * erfcl(-x / sqrtl(2.0L)); }

// Q(p) for 0 < p <= 1/2 by bisection: Phi is increasing; 200 halvings reach the
// long-double resolution of the bracket [-40, 0].
long double q_lower(long double p) {
  long double lo = -40.0L, hi = 0.0L;
  for (int it = 0; it < 200; ++it) {
    const long double mid = 0.5L * (lo + hi);
    if (mid == lo || mid == hi) break;
    if (phi(mid) < p) lo = mid; else hi = mid;
  }
  return 0.5L * (lo + hi);
}

// Q(num/den), mirrored so Q(1 - p) == -Q(p) exactly.
long double q_frac(int num, int den) {
  if (2 * num > den) return -q_frac(den - num, den);
  if (2 * num == den) return 0.0L;
  return q_lower((long double)num / (long double)den);
}

uint16_t bf16_rne_host(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  const uint32_t lsb = (u >> 16) & 1u;
  return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

// Thresholds and byte tables of a table whose 16 FP32 levels are already in t->q.
void finish_tables(Nf4Tables* t);

}  // namespace

void build_nf4_tables(Nf4Tables* t) {
  const int den = 17;
  long double raw[16];
  raw[0] = q_frac(1, 2 * den);
  for (int i = 1; i < 16; ++i) raw[i] = 0.5L * (q_frac(i, den) + q_frac(i + 1, den));
  const long double neg = -raw[0];
  const long double pos = raw[15];
  for (int i = 0; i < 16; ++i) {
    long double v = (i < 8) ? raw[i] / neg : (i == 8 ? 0.0L : raw[i] / pos);
    t->q[i] = (float)v;  // one rounding, long double -> float, to nearest even
  }
  t->q[0] = -1.0f;
  t->q[8] = 0.0f;
  t->q[15] = 1.0f;
  finish_tables(t);
}

// Other first-level codebooks, for comparison with NF4 ("QLoRA: Quantize Base Weights to
// 4-Bit", Section 2 "1. 4-bit NormalFloat", against standard INT4 and FP4):
//   INT4 : 16 evenly spaced levels -1 + 2 i / 15 (both ends exact, no zero level);
//   FP4  : the E2M1 magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 with both signs, over 6, so the ends
//          are +-1; +0 and -0 are one level and the 16th entry repeats +1 (never nearest first).
// Each level is its double value rounded once to FP32.
void build_codebook_tables(int codebook, Nf4Tables* t) {
  if (codebook == 1) {
    for (int i = 0; i < 16; ++i) t->q[i] = (float)((2.0 * i - 15.0) / 15.0);
  } else if (codebook == 2) {
    const double mags[7] = {6.0, 4.0, 3.0, 2.0, 1.5, 1.0, 0.5};
    for (int i = 0; i < 7; ++i) t->q[i] = (float)(-mags[i] / 6.0);
    t->q[7] = 0.0f;
    for (int i = 0; i < 7; ++i) t->q[8 + i] = (float)(mags[6 - i] / 6.0);
    t->q[15] = 1.0f;
  } else {
    build_nf4_tables(t);
    return;
  }
  finish_tables(t);
}

namespace {

void finish_tables(Nf4Tables* t) {
  // Decision thresholds: the exact midpoint of two FP32 levels is exact in double;
  // round it down to FP32 so that "rho > thr" equals "rho is nearer the upper level"
  // with ties going to the lower level.
  for (int k = 0; k < 15; ++k) {
    const double m = 0.5 * ((double)t->q[k] + (double)t->q[k + 1]);
    float f = (float)m;
    if ((double)f > m) f = std::nextafterf(f, -INFINITY);
    t->thr[k] = f;
  }
  // Byte tables of the unscaled BF16 levels for the byte-permute decoder.
  for (int w = 0; w < 4; ++w) {
    uint32_t lo = 0, hi = 0;
    for (int b = 0; b < 4; ++b) {
      const uint16_t h = bf16_rne_host(t->q[4 * w + b]);
      lo |= (uint32_t)(h & 0xFFu) << (8 * b);
      hi |= (uint32_t)(h >> 8) << (8 * b);
    }
    t->lut_lo[w] = lo;
    t->lut_hi[w] = hi;
  }
}

struct AllTables {
  Nf4Tables t[3];
  AllTables() {
    for (int c = 0; c < 3; ++c) build_codebook_tables(c, &t[c]);
  }
};

}  // namespace

const Nf4Tables& codebook_tables(int codebook) {
  static const AllTables all;
  return all.t[(codebook >= 0 && codebook < 3) ? codebook : 0];
}

const Nf4Tables& nf4_tables() { return codebook_tables(0); }

}  // namespace qlora
