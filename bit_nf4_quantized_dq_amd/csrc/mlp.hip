// Element-wise steps of the MLP block whose three projections (gate, up, down) are all
// NF4 + LoRA linears ("QLoRA -- Fine-Tuning a 65B Model on One GPU", "Seeing it in code":
// adapters on every linear, gate_proj, up_proj and down_proj among them; gradient
// checkpointing on, as "QLoRA: Quantize Base Weights to 4-Bit", "In production", also asks).
// The pages name the projections but not the activation between them; the one the names
// denote is the SiLU-gated product
//   H = silu(G) * U,  silu(g) = g * sigmoid(g),  G = gate(X), U = up(X),  Y = down(H)
// and its derivative
//   dG = dH * U * sigmoid(G) * (1 + G * (1 - sigmoid(G))),   dU = dH * silu(G).
// Inputs and outputs are BF16; each value is computed in FP32 from the exact BF16 inputs and
// rounded once (RNE).  The two input gradients of the block (through gate and through up)
// are added by k_add_bf16.  All three kernels are HBM-bound: one thread per 8 consecutive
// values, 16-byte loads and stores, grid-stride.
#include <algorithm>

#include "qlora_device.h"
#include "qlora_host.h"

namespace qlora {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ void unpack8(const uint4 v, float f[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16lo_to_f32(w[i]);
    f[2 * i + 1] = bf16hi_to_f32(w[i]);
  }
}
__device__ __forceinline__ uint4 pack8(const float f[8]) {
  return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
}
__device__ __forceinline__ float sigmoid(float g) { return 1.f / (1.f + expf(-g)); }

__global__ __launch_bounds__(kThreads) void k_swiglu_fwd(const uint4* __restrict__ G, const uint4* __restrict__ U,
                                                         uint4* __restrict__ H, int64_t n8) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n8; i += stride) {
    float g[8], u[8], h[8];
    unpack8(G[i], g);
    unpack8(U[i], u);
#pragma unroll
    for (int k = 0; k < 8; ++k) h[k] = g[k] * sigmoid(g[k]) * u[k];
    H[i] = pack8(h);
  }
}

__global__ __launch_bounds__(kThreads) void k_swiglu_bwd(const uint4* __restrict__ dH, const uint4* __restrict__ G,
                                                         const uint4* __restrict__ U, uint4* __restrict__ dG,
                                                         uint4* __restrict__ dU, int64_t n8) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n8; i += stride) {
    float dh[8], g[8], u[8], dg[8], du[8];
    unpack8(dH[i], dh);
    unpack8(G[i], g);
    unpack8(U[i], u);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float sg = sigmoid(g[k]);
      du[k] = dh[k] * (g[k] * sg);
      dg[k] = dh[k] * u[k] * (sg * (1.f + g[k] * (1.f - sg)));
    }
    dG[i] = pack8(dg);
    dU[i] = pack8(du);
  }
}

__global__ __launch_bounds__(kThreads) void k_add_bf16(const uint4* __restrict__ a, const uint4* __restrict__ b,
                                                       uint4* __restrict__ c, int64_t n8) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n8; i += stride) {
    float x[8], y[8];
    unpack8(a[i], x);
    unpack8(b[i], y);
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] += y[k];
    c[i] = pack8(x);
  }
}

unsigned grid_for(int64_t n8) {
  const int64_t blocks = (n8 + kThreads - 1) / kThreads;
  return (unsigned)(blocks < 4096 ? (blocks > 0 ? blocks : 1) : 4096);
}

__global__ __launch_bounds__(kThreads) void k_zero_words(unsigned int* __restrict__ p, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) p[i] = 0u;
}

}  // namespace

// The counter head of a workspace (qlora_workspace_init): a fill kernel rather than a memset,
// so that it may sit in a captured graph.
hipError_t launch_zero_words(unsigned int* p, int64_t n, hipStream_t st) {
  const int64_t blocks = std::min<int64_t>((n + kThreads - 1) / kThreads, 1024);
  hipLaunchKernelGGL(k_zero_words, dim3((unsigned)std::max<int64_t>(blocks, 1)), dim3(kThreads), 0, st, p, n);
  return hipGetLastError();
}

hipError_t launch_swiglu_fwd(const uint16_t* G, const uint16_t* U, uint16_t* H, int64_t n, hipStream_t st) {
  if (n % 8 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_swiglu_fwd, dim3(grid_for(n / 8)), dim3(kThreads), 0, st, reinterpret_cast<const uint4*>(G),
                     reinterpret_cast<const uint4*>(U), reinterpret_cast<uint4*>(H), n / 8);
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const uint16_t* dH, const uint16_t* G, const uint16_t* U, uint16_t* dG, uint16_t* dU,
                             int64_t n, hipStream_t st) {
  if (n % 8 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_swiglu_bwd, dim3(grid_for(n / 8)), dim3(kThreads), 0, st, reinterpret_cast<const uint4*>(dH),
                     reinterpret_cast<const uint4*>(G), reinterpret_cast<const uint4*>(U), reinterpret_cast<uint4*>(dG),
                     reinterpret_cast<uint4*>(dU), n / 8);
  return hipGetLastError();
}

hipError_t launch_add_bf16(const uint16_t* a, const uint16_t* b, uint16_t* c, int64_t n, hipStream_t st) {
  if (n % 8 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_add_bf16, dim3(grid_for(n / 8)), dim3(kThreads), 0, st, reinterpret_cast<const uint4*>(a),
                     reinterpret_cast<const uint4*>(b), reinterpret_cast<uint4*>(c), n / 8);
  return hipGetLastError();
}

}  // namespace qlora
