// Standalone dequantization to BF16, bit-exact (the decode steps are in decode_tiles.h).
// It runs the same per-block scaled byte-permute decoder as the fused forward GEMM, so its
// bit-exact check against the oracle covers that decoder too.
#include "decode_tiles.h"
#include "qlora_host.h"

namespace qlora {
namespace {

constexpr int kThreads = 256;

// kDecWords 8-weight code words per thread.
template <int DQ>
__global__ __launch_bounds__(kThreads) void k_dequant(const uint32_t* __restrict__ codes,
                                                      const uint8_t* __restrict__ code8,
                                                      const float* __restrict__ c2s,
                                                      const float* __restrict__ mu,
                                                      uint4* __restrict__ out, int64_t n_words,
                                                      Nf4Tables T) {
  decode_words<DQ, kThreads>(codes, code8, c2s, mu, out, blockIdx.x, threadIdx.x, n_words, T);
}

// The transposed copy w_hat^T [K, N]: 128 rows x 4 blocks per workgroup (decode_pairs_t).
template <int DQ>
__global__ __launch_bounds__(kThreads) void k_dequant_t(const uint32_t* __restrict__ codes,
                                                        const uint8_t* __restrict__ code8,
                                                        const float* __restrict__ c2s,
                                                        const float* __restrict__ mu,
                                                        uint16_t* __restrict__ out, int64_t N, int64_t K,
                                                        Nf4Tables T) {
  decode_pairs_t<DQ, kThreads>(codes, code8, c2s, mu, out, N, K, T, blockIdx.y, blockIdx.x, threadIdx.x);
}

}  // namespace

hipError_t launch_dequant_t(const uint32_t* codes, const uint8_t* code8, const float* c2s,
                            const float* mu, int64_t N, int64_t K, uint16_t* out, const Nf4Tables& T, int dq,
                            hipStream_t s) {
  dim3 grid((unsigned)((K / 64 + kThreads / 64 - 1) / (kThreads / 64)), (unsigned)((N + kTRows - 1) / kTRows));
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
  const int64_t grid = (n_words + kThreads * kDecWords - 1) / (kThreads * kDecWords);
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
