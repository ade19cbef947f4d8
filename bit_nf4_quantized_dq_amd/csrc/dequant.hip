// Standalone dequantization to BF16, bit-exact:
//   c1_hat = fl32(fl32(E4M3(code8) * c2s) + mu)      (undo DQ: "QLoRA: Quantize Base
//            Weights to 4-Bit", Section 2 "2. Double Quantization"; the comparison formats
//            read E5M2 or a signed byte instead, or the FP32 constant itself)
//   w_hat  = bf16(fl32(q[code] * c1_hat))             (lookup times constant: "QLoRA --
//            Fine-Tuning a 65B Model on One GPU", "Quantization in one paragraph")
// It runs the same per-block scaled byte-permute decoder as the fused forward GEMM, so
// its bit-exact check against the oracle covers that decoder too.
#include "qlora_device.h"
#include "qlora_host.h"

namespace qlora {
namespace {

constexpr int kThreads = 256;

// The stored constant of block blk and the block's recovered c1 (DQ: second-level format).
template <int DQ>
__device__ __forceinline__ float load_scale(const uint8_t* __restrict__ code8, const float* __restrict__ c2s,
                                            const float* __restrict__ mu, int64_t blk) {
  if (DQ == kDqNone) return reinterpret_cast<const float*>(code8)[blk];
  return block_scale_fmt<DQ>(code8[blk], c2s[blk >> 8], mu[0]);
}

template <int DQ>
__global__ __launch_bounds__(kThreads) void k_dequant(const uint32_t* __restrict__ codes,
                                                      const uint8_t* __restrict__ code8,
                                                      const float* __restrict__ c2s,
                                                      const float* __restrict__ mu,
                                                      uint4* __restrict__ out, int64_t n_words,
                                                      Nf4Tables T) {
  const int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (g >= n_words) return;
  const int64_t blk = g >> 3;
  const float c = load_scale<DQ>(code8, c2s, mu, blk);
  Lut L;
  build_scaled_lut(T, c, L);
  uint32_t w[4];
  decode8(codes[g], L, w);
  out[g] = make_uint4(w[0], w[1], w[2], w[3]);
}

// Transposed copy w_hat^T [K, N] (the operand layout of the dX product, whose reduction
// runs over N).  A workgroup decodes a 64 (n) x 256 (k) tile -- thread t one 64-weight block
// of row n0 + (t & 63) with the per-block scaled table -- into LDS, then writes the tile
// transposed: each item is a pair of rows k, k+1 times 8 consecutive n (two 16-byte stores).
// The LDS tile is [64][129] dwords (a dword = two k-neighbours), so the decode writes (one
// dword column across 64 rows) and the transposed reads (8 rows 8c+i across lanes c) both
// spread over distinct banks.
constexpr int kTN = 64, kTK = 256, kTPitch = kTK / 2 + 1;

template <int DQ>
__global__ __launch_bounds__(kThreads) void k_dequant_t(const uint32_t* __restrict__ codes,
                                                        const uint8_t* __restrict__ code8,
                                                        const float* __restrict__ c2s,
                                                        const float* __restrict__ mu,
                                                        uint16_t* __restrict__ out, int64_t N, int64_t K,
                                                        Nf4Tables T) {
  __shared__ uint32_t tile[kTN * kTPitch];
  const int t = threadIdx.x;
  const int64_t n0 = (int64_t)blockIdx.y * kTN, k0 = (int64_t)blockIdx.x * kTK;
  const int nl = t & 63, b = t >> 6;
  const int64_t n = n0 + nl, kb = k0 / 64 + b, nb_row = K / 64;
  uint32_t o[32];
  if (n < N && kb < nb_row) {
    const int64_t blk = n * nb_row + kb;
    Lut L;
    build_scaled_lut(T, load_scale<DQ>(code8, c2s, mu, blk), L);
    const uint4* wp = reinterpret_cast<const uint4*>(codes + blk * 8);
    const uint4 w0 = wp[0], w1 = wp[1];
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
    const int item = t + kThreads * q;
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

}  // namespace

hipError_t launch_dequant_t(const uint32_t* codes, const uint8_t* code8, const float* c2s,
                            const float* mu, int64_t N, int64_t K, uint16_t* out, const Nf4Tables& T, int dq,
                            hipStream_t s) {
  dim3 grid((unsigned)((K + kTK - 1) / kTK), (unsigned)((N + kTN - 1) / kTN));
  LaunchTimer t(8, s);
  auto go = [&](auto kern) {
    hipExtLaunchKernelGGL(kern, grid, dim3(kThreads), 0, s, t.start, t.stop, 0, codes, code8, c2s, mu, out, N, K, T);
  };
  if (dq == kDqE5M2) go(k_dequant_t<kDqE5M2>);
  else if (dq == kDqInt8) go(k_dequant_t<kDqInt8>);
  else if (dq == kDqNone) go(k_dequant_t<kDqNone>);
  else go(k_dequant_t<kDqE4M3>);
  return hipGetLastError();
}

hipError_t launch_dequant(const uint32_t* codes, const uint8_t* code8, const float* c2s,
                          const float* mu, uint16_t* out, int64_t n_words, const Nf4Tables& T, int dq,
                          hipStream_t s) {
  const int64_t grid = (n_words + kThreads - 1) / kThreads;
  LaunchTimer t(2, s);
  auto go = [&](auto kern) {
    hipExtLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), 0, s, t.start, t.stop, 0, codes, code8, c2s, mu,
                          reinterpret_cast<uint4*>(out), n_words, T);
  };
  if (dq == kDqE5M2) go(k_dequant<kDqE5M2>);
  else if (dq == kDqInt8) go(k_dequant<kDqInt8>);
  else if (dq == kDqNone) go(k_dequant<kDqNone>);
  else go(k_dequant<kDqE4M3>);
  return hipGetLastError();
}

}  // namespace qlora
