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
// over N), one 64 (n) x 256 (k) tile per 256 threads: thread t decodes one 64-weight block of
// row n0 + (t & 63) with the per-block scaled table into LDS, then the tile is written
// transposed, each item a pair of rows k, k+1 times 8 consecutive n (two 16-byte stores).
// The LDS tile is [64][129] dwords (a dword = two k-neighbours), so the decode writes (one
// dword column across 64 rows) and the transposed reads (8 rows 8c+i across lanes c) both
// spread over distinct banks.  Contains a workgroup barrier: every thread of the workgroup
// must call it.  Tiles past the weight decode zeros and store nothing.
constexpr int kTN = 64, kTK = 256, kTPitch = kTK / 2 + 1;
constexpr int kTileLdsBytes = kTN * kTPitch * 4;

template <int DQ>
__device__ __forceinline__ void decode_tile_t(const uint32_t* __restrict__ codes, const uint8_t* __restrict__ code8,
                                              const float* __restrict__ c2s, const float* __restrict__ mu,
                                              uint16_t* __restrict__ out, int64_t N, int64_t K, const Nf4Tables& T,
                                              int64_t tile_k, int64_t tile_n, int t, uint32_t* tile) {
  const int64_t n0 = tile_n * kTN, k0 = tile_k * kTK;
  const int nl = t & 63, b = t >> 6;
  const int64_t n = n0 + nl, kb = k0 / 64 + b, nb_row = K / 64;
  uint32_t o[32];
  if (n < N && kb < nb_row) {
    const int64_t blk = n * nb_row + kb;
    // the block's codes first (raw buffer loads, issued before the constant's decode and its
    // branch, as in decode_words)
    const rsrc_t rc = make_rsrc(codes, (int64_t)0xFFFFFFFF);
    const uint4 w0 = bload16(rc, (uint32_t)(32 * blk)), w1 = bload16(rc, (uint32_t)(32 * blk + 16));
    Lut L;
    build_scaled_lut(T, stored_c1<DQ>(code8, c2s, mu, blk), L);
    const uint32_t words[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
    for (int c = 0; c < 8; ++c) decode8(words[c], L, &o[4 * c]);
  } else {
#pragma unroll
    for (int j = 0; j < 32; ++j) o[j] = 0u;
  }
#pragma unroll
  for (int j = 0; j < 32; ++j) tile[nl * kTPitch + 32 * b + j] = o[j];
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int item = t + 256 * q;
    const int c = item & 7, p = item >> 3;  // n-chunk c (8 values), k pair p
    const int64_t k = k0 + 2 * p, nn = n0 + 8 * c;
    if (k >= K || nn >= N) continue;
    uint32_t d[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) d[i] = tile[(8 * c + i) * kTPitch + p];
    const uint4 even = make_uint4((d[0] & 0xFFFFu) | (d[1] << 16), (d[2] & 0xFFFFu) | (d[3] << 16),
                                  (d[4] & 0xFFFFu) | (d[5] << 16), (d[6] & 0xFFFFu) | (d[7] << 16));
    const uint4 odd = make_uint4((d[0] >> 16) | (d[1] & 0xFFFF0000u), (d[2] >> 16) | (d[3] & 0xFFFF0000u),
                                 (d[4] >> 16) | (d[5] & 0xFFFF0000u), (d[6] >> 16) | (d[7] & 0xFFFF0000u));
    *reinterpret_cast<uint4*>(out + k * N + nn) = even;
    *reinterpret_cast<uint4*>(out + (k + 1) * N + nn) = odd;
  }
}

}  // namespace qlora
