// AdamW step over the flat trainable adapter parameters.
//
// State per parameter, as the pages account for it: an FP32 master weight, an FP32 first
// moment and an FP32 second moment (12 bytes), beside the BF16 working weight and the BF16
// gradient ("QLoRA: Quantize Base Weights to 4-Bit", Section 1 and the optimizer term of
// Section 4; "QLoRA -- Fine-Tuning a 65B Model on One GPU", "Paged optimizers").  The update
// is the published AdamW (Loshchilov and Hutter, "Decoupled Weight Decay Regularization",
// 2019; bias correction of Kingma and Ba, "Adam", 2015), decay scaled by the learning rate:
//   theta *= 1 - lr wd;  m = b1 m + (1 - b1) g;  v = b2 v + (1 - b2) g^2;
//   theta -= (lr / (1 - b1^t)) m / (sqrt(v) / sqrt(1 - b2^t) + eps);  param = bf16(theta).
// The step-dependent scalars are formed on the host in FP64 and rounded once to FP32.
//
// The kernel is a pure stream: 14 bytes read and 14 written per parameter (28 B), so it is
// bound by HBM.  Each lane takes 4 consecutive parameters (16-byte state loads, 8-byte
// gradient loads and parameter stores); a tail of n % 4 parameters runs element by element.
#include "qlora_device.h"
#include "qlora_host.h"

namespace qlora {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ void adamw1(float& th, float& m, float& v, float g, const AdamWScalars& a) {
  th = __fmul_rn(th, a.decay);
  m = __fadd_rn(__fmul_rn(a.b1, m), __fmul_rn(a.omb1, g));
  v = __fadd_rn(__fmul_rn(a.b2, v), __fmul_rn(a.omb2, __fmul_rn(g, g)));
  const float den = __fadd_rn(__fmul_rn(__fsqrt_rn(v), a.inv_bc2_sqrt), a.eps);
  th = __fsub_rn(th, __fdiv_rn(__fmul_rn(a.step_size, m), den));
}

__global__ __launch_bounds__(kThreads) void k_adamw(float* __restrict__ master, float* __restrict__ mom1,
                                                    float* __restrict__ mom2, const uint16_t* __restrict__ grad,
                                                    uint16_t* __restrict__ param, int64_t n, AdamWScalars a) {
  const int64_t n4 = n >> 2;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n4; i += stride) {
    float4 th = reinterpret_cast<const float4*>(master)[i];
    float4 m = reinterpret_cast<const float4*>(mom1)[i];
    float4 v = reinterpret_cast<const float4*>(mom2)[i];
    const uint2 gb = reinterpret_cast<const uint2*>(grad)[i];
    adamw1(th.x, m.x, v.x, bf16lo_to_f32(gb.x), a);
    adamw1(th.y, m.y, v.y, bf16hi_to_f32(gb.x), a);
    adamw1(th.z, m.z, v.z, bf16lo_to_f32(gb.y), a);
    adamw1(th.w, m.w, v.w, bf16hi_to_f32(gb.y), a);
    reinterpret_cast<float4*>(master)[i] = th;
    reinterpret_cast<float4*>(mom1)[i] = m;
    reinterpret_cast<float4*>(mom2)[i] = v;
    if (param) reinterpret_cast<uint2*>(param)[i] = make_uint2(pack_bf16x2(th.x, th.y), pack_bf16x2(th.z, th.w));
  }
  // tail: the last n % 4 parameters, one per lane of the first workgroup
  if (blockIdx.x == 0 && threadIdx.x < (n & 3)) {
    const int64_t j = 4 * n4 + threadIdx.x;
    float th = master[j], m = mom1[j], v = mom2[j];
    adamw1(th, m, v, __uint_as_float((uint32_t)grad[j] << 16), a);
    master[j] = th;
    mom1[j] = m;
    mom2[j] = v;
    if (param) param[j] = (uint16_t)(pack_bf16x2(th, 0.f) & 0xFFFFu);
  }
}

}  // namespace

hipError_t launch_adamw(float* master, float* m, float* v, const uint16_t* grad, uint16_t* param, int64_t n,
                        const AdamWScalars& a, hipStream_t s) {
  const int64_t n4 = n >> 2;
  const int64_t want = (n4 + kThreads - 1) / kThreads;
  const unsigned grid = (unsigned)(want < 1 ? 1 : (want > 65536 ? 65536 : want));
  LaunchTimer t(10, s);
  hipExtLaunchKernelGGL(k_adamw, dim3(grid), dim3(kThreads), 0, s, t.start, t.stop, 0, master, m, v, grad, param, n, a);
  return hipGetLastError();
}

}  // namespace qlora
