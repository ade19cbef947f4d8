// Decode of the stored weight to BF16, bit-exact, as device functions shared by the
// standalone decode kernels (dequant.hip) and the launches that pair a decode with the LoRA
// down-projection (lora.hip):
//   c1_hat = fl32(fl32(E4M3(code8) * c2s) + mu)      (undo DQ: "QLoRA: Quantize Base
//            Weights to 4-Bit", Section 2 "2. Double Quantization"; the comparison formats
//            read E5M2 or a signed byte instead, or the FP32 constant itself)
//   w_hat  = bf16(fl32(q[code] * c1_hat))             (lookup times constant: "QLoRA --
//            Fine-Tuning a 65B Model on One GPU", "Quantization in one paragraph")
#pragma once

#include "qlora_device.h"

namespace qlora {

// The stored constant of block blk and the block's recovered c1 (DQ: second-level format).
template <int DQ>
__device__ __forceinline__ float stored_c1(const uint8_t* __restrict__ code8, const float* __restrict__ c2s,
                                           const float* __restrict__ mu, int64_t blk) {
  if (DQ == kDqNone) return reinterpret_cast<const float*>(code8)[blk];
  return block_scale_fmt<DQ>(code8[blk], c2s[blk >> 8], mu[0]);
}

// Code words (blk kDecWords + i) NT + t, i < kDecWords, decoded by thread t of workgroup blk
// (NT threads) into out[word] (4 dwords of BF16 pairs, element order).  The code words are
// loaded first, as raw buffer loads (the constant's decode holds a branch, and a plain load
// placed after it waited for the constant's round trip before it issued), and all of a
// thread's loads go out before its first decode: with one word per thread the decode ran as
// thousands of small workgroups that overlapped poorly with the launch it shares a grid with.
constexpr int kDecWords = 8;
template <int DQ, int NT>
__device__ __forceinline__ void decode_words(const uint32_t* __restrict__ codes, const uint8_t* __restrict__ code8,
                                             const float* __restrict__ c2s, const float* __restrict__ mu,
                                             uint4* __restrict__ out, int64_t blk, int t, int64_t n_words,
                                             const Nf4Tables& T) {
  const rsrc_t rc = make_rsrc(codes, (int64_t)0xFFFFFFFF);
  uint32_t cw[kDecWords];
  float c1[kDecWords];
  int64_t g[kDecWords];
#pragma unroll
  for (int i = 0; i < kDecWords; ++i) {
    g[i] = (blk * kDecWords + i) * NT + t;
    const bool ok = g[i] < n_words;
    cw[i] = bload4(rc, ok ? (uint32_t)(4 * g[i]) : kOOB);
    c1[i] = stored_c1<DQ>(code8, c2s, mu, ok ? g[i] >> 3 : 0);
  }
#pragma unroll
  for (int i = 0; i < kDecWords; ++i) {
    if (g[i] >= n_words) continue;
    Lut L;
    build_scaled_lut(T, c1[i], L);
    uint32_t w[4];
    decode8(cw[i], L, w);
    out[g[i]] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Transposed copy w_hat^T [K, N] (the operand layout of the dX product, whose reduction runs
// over N), without LDS: lane l of wavefront w of workgroup (gn, gk) decodes block
// kb = gk (NT / 64) + w of rows n = 128 gn + 2 l and n + 1 (the per-block scaled table, one
// per row), and for each of the block's 64 reduction indices k stores the dword
// (w_hat[n][k], w_hat[n + 1][k]) at row k of the output: the 64 lanes of a wavefront write
// 256 contiguous bytes of that row.  (A tile transposed through LDS needed 66 KB per
// workgroup, which held the launch that pairs it with G = dY B to two workgroups per CU.)
// N is even, so a row pair is whole.  Blocks past the weight store nothing.
constexpr int kTRows = 128;  // rows per workgroup (two per lane)
template <int DQ, int NT>
__device__ __forceinline__ void decode_pairs_t(const uint32_t* __restrict__ codes, const uint8_t* __restrict__ code8,
                                               const float* __restrict__ c2s, const float* __restrict__ mu,
                                               uint16_t* __restrict__ out, int64_t N, int64_t K, const Nf4Tables& T,
                                               int64_t gn, int64_t gk, int t) {
  const int lane = t & 63, w = t >> 6;
  const int64_t n = gn * kTRows + 2 * lane, nb_row = K / 64, kb = gk * (NT / 64) + w;
  if (n >= N || kb >= nb_row) return;
  const int64_t blk0 = n * nb_row + kb, blk1 = blk0 + nb_row;
  // the codes first (raw buffer loads, issued before the constants' decode and its branch,
  // as in decode_words)
  const rsrc_t rc = make_rsrc(codes, (int64_t)0xFFFFFFFF);
  const uint4 a0 = bload16(rc, (uint32_t)(32 * blk0)), a1 = bload16(rc, (uint32_t)(32 * blk0 + 16));
  const uint4 b0 = bload16(rc, (uint32_t)(32 * blk1)), b1 = bload16(rc, (uint32_t)(32 * blk1 + 16));
  Lut La, Lb;
  build_scaled_lut(T, stored_c1<DQ>(code8, c2s, mu, blk0), La);
  build_scaled_lut(T, stored_c1<DQ>(code8, c2s, mu, blk1), Lb);
  const uint32_t wa[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
  const uint32_t wb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
  uint32_t* const o = reinterpret_cast<uint32_t*>(out) + (kb * 64 * N + n) / 2;  // row k = 64 kb, column n
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    uint32_t da[4], db[4];  // dword j: elements 8c + 2j (low half) and 8c + 2j + 1 (high half)
    decode8(wa[c], La, da);
    decode8(wb[c], Lb, db);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t k = 8 * c + 2 * j;  // within the block
      o[(k * N) / 2] = __builtin_amdgcn_perm(db[j], da[j], 0x05040100u);        // (n, n + 1) at k
      o[((k + 1) * N) / 2] = __builtin_amdgcn_perm(db[j], da[j], 0x07060302u);  // (n, n + 1) at k + 1
    }
  }
}

}  // namespace qlora
