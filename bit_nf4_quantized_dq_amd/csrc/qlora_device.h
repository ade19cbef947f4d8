// Device helpers shared by the HIP kernels: the NF4 tables passed to kernels, OCP E4M3
// encode/decode, BF16 rounding, and the byte-permute decode of packed 4-bit codes.
//
// Format recap ("QLoRA -- Fine-Tuning a 65B Model on One GPU", "Quantization in one
// paragraph" and "Double quantization"; "QLoRA: Quantize Base Weights to 4-Bit", Section 2):
//   codes : 4-bit level indices; each aligned run of 8 weights e0..e7 is one 32-bit word
//           whose byte i holds e_i in its low nibble and e_{i+4} in its high nibble.
//   code8 : one OCP E4M3 byte per 64-weight block (mean-shifted, second-level scaled c1).
//   c2s   : one FP32 per 256 blocks.   mu : one FP32 per tensor.
//   c1_hat = fl32(fl32(E4M3(code8) * c2s) + mu);   w_hat = bf16(fl32(q[code] * c1_hat)).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qlora_tables.h"

namespace qlora {

constexpr int kBlock1 = 64;   // weights per absmax block
constexpr int kBlock2 = 256;  // blocks per second-level group

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8_t;   // MFMA operand
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;    // 16x16 MFMA acc
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;

// ---------------------------------------------------------------- scalar conversions

// OCP FP8 E4M3 ("E4M3FN") -> FP32, exact.  Exponent bias 7; exponent field 0 is
// subnormal (m/8 * 2^-6).  NaN (S.1111.111) never occurs in stored codes.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  const uint32_t e = (b >> 3) & 0xFu;
  const uint32_t m = b & 0x7u;
  float v;
  if (e == 0) {
    v = (float)m * 0.001953125f;  // m * 2^-9, exact
  } else {
    v = __uint_as_float(((e + 120u) << 23) | (m << 20));
  }
  return (b & 0x80u) ? -v : v;
}

// FP32 -> OCP E4M3, round to nearest, ties to even; |s| beyond 448 saturates to 448;
// the sign of zero follows the sign of s.  Written from the OCP OFP8 definition.
__device__ __forceinline__ uint32_t f32_to_e4m3(float s) {
  const uint32_t u = __float_as_uint(s);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t E = (u >> 23) & 0xFFu;
  uint32_t code;
  if (E < 121u) {
    // below the smallest normal 2^-6: subnormal grid m * 2^-9, m = RNE(|s| * 2^9) in 0..8
    const float t = __uint_as_float(u & 0x7FFFFFFFu) * 512.0f;  // exact scaling
    code = (uint32_t)__builtin_rintf(t);                          // RNE; 8 -> 0x08 (= 2^-6)
  } else {
    const uint32_t mant = u & 0x7FFFFFu;
    code = ((E - 120u) << 3) | (mant >> 20);
    const uint32_t rem = mant & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (code & 1u))) code += 1u;
    if (code > 0x7Eu) code = 0x7Eu;
  }
  return code | sign;
}

// Two FP32 -> packed BF16 pair (lo = a, hi = b), round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  typedef float f2 __attribute__((ext_vector_type(2)));
  f2 v = {a, b};
  bf2 r = __builtin_convertvector(v, bf2);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float bf16lo_to_f32(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t p) { return __uint_as_float(p & 0xFFFF0000u); }

// Recovered block constant, two separate FP32 roundings (no contraction).
__device__ __forceinline__ float block_scale(uint32_t code8, float c2s, float mu) {
  return __fadd_rn(__fmul_rn(e4m3_to_f32(code8), c2s), mu);
}

// ---------------------------------------------------------------- second-level format variants
// The format of the stored block constants (the comparison formats of "QLoRA: Quantize Base
// Weights to 4-Bit", Section 2 "2. Double Quantization", whose 8-bit format the pages call
// both a float and an integer, and FP32 constants without double quantization).
enum DqFormat : int { kDqE4M3 = 0, kDqE5M2 = 1, kDqInt8 = 2, kDqNone = 3 };

// OCP FP8 E5M2 -> FP32, exact: bias 15, 2 mantissa bits, exponent field 0 subnormal
// (m/4 * 2^-14).  Inf and NaN codes never occur in stored constants.
__device__ __forceinline__ float e5m2_to_f32(uint32_t b) {
  const uint32_t e = (b >> 2) & 0x1Fu;
  const uint32_t m = b & 0x3u;
  const float v = (e == 0) ? (float)m * 1.52587890625e-05f  // m * 2^-16, exact
                           : __uint_as_float(((e + 112u) << 23) | (m << 21));
  return (b & 0x80u) ? -v : v;
}

// FP32 -> OCP E5M2, round to nearest, ties to even; beyond 57344 to 57344; the sign of zero
// follows s.  Written from the OCP OFP8 definition, like the E4M3 encoder above.
__device__ __forceinline__ uint32_t f32_to_e5m2(float s) {
  const uint32_t u = __float_as_uint(s);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t E = (u >> 23) & 0xFFu;
  uint32_t code;
  if (E < 113u) {
    // below the smallest normal 2^-14: grid m * 2^-16, m = RNE(|s| * 2^16) in 0..4
    code = (uint32_t)__builtin_rintf(__uint_as_float(u & 0x7FFFFFFFu) * 65536.0f);
  } else {
    const uint32_t mant = u & 0x7FFFFFu;
    code = ((E - 112u) << 2) | (mant >> 21);
    const uint32_t rem = mant & 0x1FFFFFu;
    if (rem > 0x100000u || (rem == 0x100000u && (code & 1u))) code += 1u;
    if (code > 0x7Bu) code = 0x7Bu;
  }
  return code | sign;
}

// FP32 -> symmetric 8-bit integer (two's-complement byte): round half to even, clamp to +-127.
__device__ __forceinline__ uint32_t f32_to_int8(float s) {
  float q = __builtin_rintf(s);
  q = q > 127.f ? 127.f : (q < -127.f ? -127.f : q);
  return (uint32_t)(int)q & 0xFFu;
}

// Block constant of a stored entry c (the 8-bit code, or for kDqNone the FP32 bits).
template <int DQ>
__device__ __forceinline__ float block_scale_fmt(uint32_t c, float c2s, float mu) {
  if (DQ == kDqNone) return __uint_as_float(c);
  const float v = DQ == kDqE4M3 ? e4m3_to_f32(c) : (DQ == kDqE5M2 ? e5m2_to_f32(c) : (float)(int8_t)(uint8_t)c);
  return __fadd_rn(__fmul_rn(v, c2s), mu);
}

// ---------------------------------------------------------------- byte-permute LUT decode
//
// A 16-entry byte table t0..t3 (entry j at dword j/4, byte j%4) is looked up for the four
// 4-bit indices held in the bytes of `idx` (values 0..15):
//   entries 0..7  : v_perm over {t1:t0} with the index as byte selector;
//   entries 8..15 : v_perm over {t3:t2} with index ^ 8;
//   select        : byte mask 0xFF where index >= 8, from v_perm over zero sources with
//                   selector index + 5 (selectors >= 13 yield 0xFF, 5..12 yield 0x00).

__device__ __forceinline__ uint32_t nib_mask(uint32_t idx) {
  return __builtin_amdgcn_perm(0u, 0u, idx + 0x05050505u);
}

__device__ __forceinline__ uint32_t lut16(uint32_t idx, uint32_t idx8, uint32_t m,
                                          uint32_t t0, uint32_t t1, uint32_t t2, uint32_t t3) {
  const uint32_t a = __builtin_amdgcn_perm(t1, t0, idx);
  const uint32_t b = __builtin_amdgcn_perm(t3, t2, idx8);
  return (b & m) | (a & ~m);
}

struct Lut {
  uint32_t lo[4];
  uint32_t hi[4];
};

// Decode one 32-bit code word (8 weights) into 4 dwords of BF16 pairs in element order:
// out[j] = bf16(e_{2j}) | bf16(e_{2j+1}) << 16, values taken from the table `L`.
__device__ __forceinline__ void decode8(uint32_t u, const Lut& L, uint32_t out[4]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t idx = (h == 0 ? u : (u >> 4)) & 0x0F0F0F0Fu;
    const uint32_t idx8 = idx ^ 0x08080808u;
    const uint32_t m = nib_mask(idx);
    const uint32_t lo = lut16(idx, idx8, m, L.lo[0], L.lo[1], L.lo[2], L.lo[3]);
    const uint32_t hi = lut16(idx, idx8, m, L.hi[0], L.hi[1], L.hi[2], L.hi[3]);
    // bytes of lo/hi belong to elements 4h+0..4h+3; interleave to BF16 pairs
    out[2 * h + 0] = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
    out[2 * h + 1] = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
  }
}

// Build the table of bf16(fl32(q[j] * c)) for a block constant c (bit-exact decode).
__device__ __forceinline__ void build_scaled_lut(const Nf4Tables& T, float c, Lut& L) {
  uint32_t p[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) p[t] = pack_bf16x2(__fmul_rn(T.q[2 * t], c), __fmul_rn(T.q[2 * t + 1], c));
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    L.lo[w] = __builtin_amdgcn_perm(p[2 * w + 1], p[2 * w], 0x06040200u);
    L.hi[w] = __builtin_amdgcn_perm(p[2 * w + 1], p[2 * w], 0x07050301u);
  }
}

__device__ __forceinline__ void load_unscaled_lut(const Nf4Tables& T, Lut& L) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    L.lo[w] = T.lut_lo[w];
    L.hi[w] = T.lut_hi[w];
  }
}

// NF4 code of one ratio rho = w / c1 (c1 > 0): the number of thresholds below rho.
// The thresholds ascend, so the count of those below rho is found by a 4-step binary
// search: at step s the candidate threshold is thr[c + 2^(3-s) - 1] for the bits c found so
// far, chosen among constants with selects.  Same result as counting all 15 (also for NaN:
// every comparison is false).
__device__ __forceinline__ uint32_t nf4_code(float rho, const Nf4Tables& T) {
  const bool b3 = rho > T.thr[7];
  const bool b2 = rho > (b3 ? T.thr[11] : T.thr[3]);
  const float t1a = b2 ? T.thr[13] : T.thr[9], t1b = b2 ? T.thr[5] : T.thr[1];
  const bool b1 = rho > (b3 ? t1a : t1b);
  const uint32_t c3 = (b3 ? 8u : 0u) | (b2 ? 4u : 0u) | (b1 ? 2u : 0u);
  // thr[c3] for c3 in {0, 2, ..., 14}
  const float u0 = b1 ? T.thr[2] : T.thr[0], u1 = b1 ? T.thr[6] : T.thr[4];
  const float u2 = b1 ? T.thr[10] : T.thr[8], u3 = b1 ? T.thr[14] : T.thr[12];
  const float v0 = b2 ? u1 : u0, v1 = b2 ? u3 : u2;
  const bool b0 = rho > (b3 ? v1 : v0);
  return c3 | (b0 ? 1u : 0u);
}

// ---------------------------------------------------------------- buffer loads
// Raw buffer loads: an offset at or beyond the descriptor's byte count returns zeros, so
// ragged tiles need no branches.  One descriptor covers at most 4 GiB from its base.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOOB = 0xFFFFFFFFu;  // an offset that is always out of range

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const uint32_t n = bytes <= 0 ? 0u : (bytes >= (int64_t)0xFFFFFFFF ? 0xFFFFFFFFu : (uint32_t)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)n, 0x00020000);
}
__device__ __forceinline__ uint4 bload16(rsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint2 bload8(rsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
  return make_uint2(v[0], v[1]);
}
__device__ __forceinline__ uint32_t bload4(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}
__device__ __forceinline__ uint32_t bload1(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, (int)off, 0, 0);
}

// ---------------------------------------------------------------- MFMA

__device__ __forceinline__ f32x4_t mfma16x16x32(const bf16x8_t& a, const bf16x8_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint32_t v[4]) {
  u32x4_t t = {v[0], v[1], v[2], v[3]};
  return __builtin_bit_cast(bf16x8_t, t);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& v) {
  u32x4_t t = {v.x, v.y, v.z, v.w};
  return __builtin_bit_cast(bf16x8_t, t);
}

// ---------------------------------------------------------------- wavefront sums

// Sum over the 64 lanes in a fixed order, the same in every lane (all 64 lanes must be active):
// within each row of 16 lanes by DPP (lane pairs, then quads, half rows and rows, each step
// adding the mirrored partner, so both partners form the same sum), then the four row sums
// in order.
template <int kCtrl>
__device__ __forceinline__ float dpp_partner(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_partner<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v += dpp_partner<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v += dpp_partner<0x141>(v);  // row_half_mirror
  v += dpp_partner<0x140>(v);  // row_mirror
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return ((r0 + r1) + r2) + r3;
}

}  // namespace qlora
