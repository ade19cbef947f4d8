// Quantize kernels: absmax NF4 with double-quantized block constants.
//
// Pass 1 ("QLoRA -- Fine-Tuning a 65B Model on One GPU", "Quantization in one paragraph"):
//   per block of 64 consecutive row-major weights, c1 = max |w|; each weight becomes the
//   index of the NF4 level nearest to fl32(w / c1) (ties to the lower level; all-zero
//   blocks take the zero level).  The exact sum of all c1 is gathered for the mean as
//   integer mantissa sums per FP32 exponent (commutative, so bit-reproducible).
// Pass 2 ("QLoRA: Quantize Base Weights to 4-Bit", Section 2 "2. Double Quantization";
//   "QLoRA -- Fine-Tuning a 65B Model on One GPU", "Double quantization"): the constants
//   are centred on their mean mu and quantized to 8-bit floats in groups of 256 with one
//   FP32 constant per group: c2s = fl32(max|c1 - mu| / 448), code8 = E4M3(fl32(d / c2s)).
//   The comparison formats swap E4M3 for E5M2 (top 57344) or a symmetric 8-bit integer (top
//   127); without double quantization pass 1 writes c1 straight into the constant buffer.
//
// Memory layout: W FP32 or BF16 [d_out*d_in] is read as 8-value words (one packed code word
// each); a wavefront covers 8 blocks of W with 16-byte lane loads.  A BF16 checkpoint (the
// 16-bit form a model ships in, and the merged export) is quantized as its exact FP32 values.
#include <cmath>

#include "qlora_device.h"
#include "qlora_host.h"

namespace qlora {
namespace {

constexpr int kThreads = 256;

// The pass is bound by its VALU work (a wave64 instruction takes 4 cycles of a 16-lane SIMD),
// so the two per-weight steps are written for few instructions, with the same results:
//
// - The ratio rho = fl32(w / c1).  The correctly rounded division is a 10-instruction
//   sequence per weight.  The block's 64 weights share c1, so each lane takes y = fl32(1 / c1)
//   once (correctly rounded) and then, per weight, q = fl32(w y) followed by two corrections
//   q <- fl32(q + fl32(w - c1 q) y), each a fused multiply-add rounded once: five instructions.
//   After the first correction q is within one ulp of w / c1, and Markstein's theorem (a
//   reciprocal within half an ulp and a quotient within one ulp give an exact remainder and a
//   correctly rounded corrected quotient) makes the second one exactly fl32(w / c1).  The
//   theorem needs no underflow or overflow on the way, which holds for 2^-40 <= c1 <= 2^100:
//   y stays normal, a remainder is a multiple of ulp(q) ulp(c1) >= 2^-149 once |q| >= 2^-60,
//   and a smaller |q| lies below every threshold's magnitude (at least 2^-50, checked on the
//   host), where any q in that range has the code of 0.  Other blocks (and codebooks with a
//   threshold that close to 0) keep the correctly rounded division.
// - The code, the number of the 15 ascending thresholds below rho, by the same 4-step binary
//   search as everywhere else, with the thresholds of steps 2-4 read from LDS at an address
//   that the steps update (3 instructions a step) instead of picked among constants.
template <int kCtrl>
__device__ __forceinline__ float dpp_max(float v) {
  return fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false)));
}
__device__ __forceinline__ float lds_f32(const float* base, uint32_t byte_off) {
  return *reinterpret_cast<const float*>(reinterpret_cast<const char*>(base) + byte_off);
}
// thr: the 15 thresholds in LDS; t7 = thr[7].  Step s reads thr at byte offset a = 4 (c + 2^(3-s) - 1)
// for the bits c found so far, so a moves by +-2^(4-s) bytes with each decision.
__device__ __forceinline__ uint32_t code_lds(float rho, const float* thr, float t7) {
  uint32_t a = rho > t7 ? 44u : 12u;  // thr[11] or thr[3]
  a += rho > lds_f32(thr, a) ? 8u : (uint32_t)-8;
  a += rho > lds_f32(thr, a) ? 4u : (uint32_t)-4;
  return (a >> 2) + (rho > lds_f32(thr, a) ? 1u : 0u);
}

// W is FP32 (BF = false: two 16-byte loads per word) or BF16 (BF = true: one 16-byte load
// per word, each value widened exactly to FP32).
// Grid-stride over code words: a workgroup takes words w, w + stride, ... (stride = grid x
// 256), so its LDS histogram gathers many blocks and the global histogram receives one
// atomic per non-empty bin per workgroup.  The constants of a tensor share a few exponents,
// so one atomic per block would pile onto the same few addresses.
// fast: the codebook allows the reciprocal form (every threshold finite, |t| >= 2^-50).
template <bool BF>
__global__ __launch_bounds__(kThreads) void k_quant_pass1(const void* __restrict__ W,
                                                          uint32_t* __restrict__ codes,
                                                          float* __restrict__ c1_out,
                                                          unsigned long long* __restrict__ hist,
                                                          int* __restrict__ flag, int64_t n_words,
                                                          Nf4Tables T, int32_t fast) {
  __shared__ unsigned long long sh_hist[256];
  __shared__ float s_thr[16];
  sh_hist[threadIdx.x] = 0ull;
  if (threadIdx.x < 15) s_thr[threadIdx.x] = T.thr[threadIdx.x];
  __syncthreads();

  bool any_bad = false;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  // g0 is the same for every thread of the workgroup, so the 8-lane shuffles see whole blocks
  for (int64_t g0 = (int64_t)blockIdx.x * kThreads; g0 < n_words; g0 += stride) {
    const int64_t g = g0 + threadIdx.x;  // one code word = 8 weights
    const bool active = g < n_words;     // n_words is a multiple of 8, so whole blocks are active
    float v[8];
    if (active && BF) {
      const uint4 a = static_cast<const uint4*>(W)[g];
      const uint32_t p[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = bf16lo_to_f32(p[i]);
        v[2 * i + 1] = bf16hi_to_f32(p[i]);
      }
    } else if (active) {
      const float4 a = static_cast<const float4*>(W)[2 * g];
      const float4 b = static_cast<const float4*>(W)[2 * g + 1];
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0.f;
    }
    bool bad = false;
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      bad |= !__builtin_isfinite(v[i]);
      mx = fmaxf(mx, fabsf(v[i]));
    }
    // absmax over the 8 lanes of one 64-weight block (lanes 8j..8j+7, a half row)
    mx = dpp_max<0xB1>(mx);   // quad_perm [1, 0, 3, 2]
    mx = dpp_max<0x4E>(mx);   // quad_perm [2, 3, 0, 1]
    mx = dpp_max<0x141>(mx);  // row_half_mirror

    uint32_t c[8];
    if (fast && mx >= 0x1p-40f && mx <= 0x1p100f) {
      const float y = __fdiv_rn(1.f, mx);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float q = v[i] * y;
        q = __builtin_fmaf(__builtin_fmaf(-q, mx, v[i]), y, q);
        q = __builtin_fmaf(__builtin_fmaf(-q, mx, v[i]), y, q);
        c[i] = code_lds(q, s_thr, T.thr[7]);
      }
    } else if (mx > 0.f) {
#pragma unroll
      for (int i = 0; i < 8; ++i) c[i] = nf4_code(__fdiv_rn(v[i], mx), T);
    } else {
      const uint32_t z = nf4_code(0.f, T);  // the level nearest 0, ties low (8 for NF4)
#pragma unroll
      for (int i = 0; i < 8; ++i) c[i] = z;
    }
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) word |= (c[i] | (c[i + 4] << 4)) << (8 * i);

    if (active) {
      codes[g] = word;
      if ((threadIdx.x & 7) == 0 && !bad) {
        c1_out[g >> 3] = mx;
        const uint32_t bits = __float_as_uint(mx);
        const uint32_t e = bits >> 23;  // mx >= 0
        const uint32_t bin = e ? e : 1u;
        const unsigned long long m = (unsigned long long)((bits & 0x7FFFFFu) | (e ? 0x800000u : 0u));
        if (m) atomicAdd(&sh_hist[bin], m);
      }
    }
    any_bad |= bad && active;
  }
  if (__any(any_bad)) {
    if ((threadIdx.x & 63) == 0) atomicOr(flag, 1);
  }
  __syncthreads();
  const unsigned long long h = sh_hist[threadIdx.x];
  if (h) atomicAdd(&hist[(blockIdx.x % kHistCopies) * 256 + threadIdx.x], h);
}

// Copy 0 of the exponent sums += copies 1 .. kHistCopies - 1 (integer adds: exact, and the
// order does not matter).  One workgroup, one bin per thread.
__global__ __launch_bounds__(kThreads) void k_hist_fold(unsigned long long* __restrict__ hist) {
  unsigned long long s = 0;
  for (int c = 0; c < kHistCopies; ++c) s += hist[c * 256 + threadIdx.x];
  hist[threadIdx.x] = s;
}

// One wavefront per group of 256 constants; lane l owns constants 4l..4l+3 of the group.
// DQ selects the 8-bit format: E4M3 (top 448), E5M2 (top 57344) or INT8 (top 127).
template <int DQ>
__global__ __launch_bounds__(kThreads) void k_quant_pass2(const float* __restrict__ c1, float mu,
                                                          uint8_t* __restrict__ code8,
                                                          float* __restrict__ c2s,
                                                          float* __restrict__ mu_out,
                                                          int64_t n_blocks) {
  const int lane = threadIdx.x & 63;
  const int64_t grp = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int64_t n_groups = (n_blocks + kBlock2 - 1) / kBlock2;
  if (blockIdx.x == 0 && threadIdx.x == 0) *mu_out = mu;
  if (grp >= n_groups) return;  // whole wavefront leaves together
  const int64_t base = grp * kBlock2 + 4 * lane;
  float d[4];
  float m = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const bool ok = base + j < n_blocks;
    d[j] = ok ? __fsub_rn(c1[base + j], mu) : 0.f;
    m = fmaxf(m, fabsf(d[j]));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  const float top = DQ == kDqE4M3 ? 448.0f : (DQ == kDqE5M2 ? 57344.0f : 127.0f);
  const float c2 = __fdiv_rn(m, top);
  uint32_t q[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float t = __fdiv_rn(d[j], c2);
    q[j] = (c2 > 0.f) ? (DQ == kDqE4M3 ? f32_to_e4m3(t) : (DQ == kDqE5M2 ? f32_to_e5m2(t) : f32_to_int8(t))) : 0u;
  }
  if (base + 3 < n_blocks && (base & 3) == 0) {
    *reinterpret_cast<uint32_t*>(code8 + base) = q[0] | (q[1] << 8) | (q[2] << 16) | (q[3] << 24);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (base + j < n_blocks) code8[base + j] = (uint8_t)q[j];
  }
  if (lane == 0) c2s[grp] = c2;
}

__global__ __launch_bounds__(kThreads) void k_e4m3_encode(const float* __restrict__ in,
                                                          uint8_t* __restrict__ out, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i < n) out[i] = (uint8_t)f32_to_e4m3(in[i]);
}

}  // namespace

hipError_t launch_quant_pass1(const void* W, bool w_bf16, uint32_t* codes, float* c1, unsigned long long* hist,
                              int* flag, int64_t n_words, const Nf4Tables& T, hipStream_t s) {
  // 2048 workgroups of 256 threads fill the chip (8 per CU); larger tensors loop
  const int64_t grid = std::min<int64_t>((n_words + kThreads - 1) / kThreads, 2048);
  int32_t fast = 1;  // every threshold finite and at least 2^-50 away from 0
  for (int k = 0; k < 15; ++k)
    if (!(std::fabs(T.thr[k]) >= 0x1p-50f && std::fabs(T.thr[k]) <= 0x1p100f)) fast = 0;
  LaunchTimer t(0, s);
  if (w_bf16)
    hipExtLaunchKernelGGL(k_quant_pass1<true>, dim3((unsigned)grid), dim3(kThreads), 0, s, t.start, t.stop, 0, W, codes,
                          c1, hist, flag, n_words, T, fast);
  else
    hipExtLaunchKernelGGL(k_quant_pass1<false>, dim3((unsigned)grid), dim3(kThreads), 0, s, t.start, t.stop, 0, W,
                          codes, c1, hist, flag, n_words, T, fast);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_hist_fold, dim3(1), dim3(kThreads), 0, s, hist);
  return hipGetLastError();
}

hipError_t launch_quant_pass2(const float* c1, float mu, uint8_t* code8, float* c2s, float* mu_out,
                              int64_t n_blocks, int dq, hipStream_t s) {
  const int64_t n_groups = (n_blocks + kBlock2 - 1) / kBlock2;
  const int64_t grid = (n_groups + 3) / 4;
  LaunchTimer t(1, s);
  auto go = [&](auto kern) {
    hipExtLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), 0, s, t.start, t.stop, 0, c1, mu, code8, c2s, mu_out,
                          n_blocks);
  };
  if (dq == kDqE5M2) go(k_quant_pass2<kDqE5M2>);
  else if (dq == kDqInt8) go(k_quant_pass2<kDqInt8>);
  else go(k_quant_pass2<kDqE4M3>);
  return hipGetLastError();
}

hipError_t launch_e4m3_encode(const float* in, uint8_t* out, int64_t n, hipStream_t s) {
  const int64_t grid = (n + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(k_e4m3_encode, dim3((unsigned)grid), dim3(kThreads), 0, s, in, out, n);
  return hipGetLastError();
}

}  // namespace qlora
