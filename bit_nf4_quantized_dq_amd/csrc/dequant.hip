// Standalone dequantization to BF16, bit-exact:
//   c1_hat = fl32(fl32(E4M3(code8) * c2s) + mu)      (undo DQ: "QLoRA: Quantize Base
//            Weights to 4-Bit", Section 2 "2. Double Quantization")
//   w_hat  = bf16(fl32(q[code] * c1_hat))             (lookup times constant: "QLoRA --
//            Fine-Tuning a 65B Model on One GPU", "Quantization in one paragraph")
// It runs the same per-block scaled byte-permute decoder as the fused forward GEMM, so
// its bit-exact check against the oracle covers that decoder too.
#include "qlora_device.h"
#include "qlora_host.h"

namespace qlora {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void k_dequant(const uint32_t* __restrict__ codes,
                                                      const uint8_t* __restrict__ code8,
                                                      const float* __restrict__ c2s,
                                                      const float* __restrict__ mu,
                                                      uint4* __restrict__ out, int64_t n_words,
                                                      Nf4Tables T) {
  const int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (g >= n_words) return;
  const int64_t blk = g >> 3;
  const float c = block_scale(code8[blk], c2s[blk >> 8], mu[0]);
  Lut L;
  build_scaled_lut(T, c, L);
  uint32_t w[4];
  decode8(codes[g], L, w);
  out[g] = make_uint4(w[0], w[1], w[2], w[3]);
}

}  // namespace

hipError_t launch_dequant(const uint32_t* codes, const uint8_t* code8, const float* c2s,
                          const float* mu, uint16_t* out, int64_t n_words, const Nf4Tables& T,
                          hipStream_t s) {
  const int64_t grid = (n_words + kThreads - 1) / kThreads;
  LaunchTimer t(2, s);
  hipLaunchKernelGGL(k_dequant, dim3((unsigned)grid), dim3(kThreads), 0, s, codes, code8, c2s, mu,
                     reinterpret_cast<uint4*>(out), n_words, T);
  return hipGetLastError();
}

}  // namespace qlora
