// Weight-streaming forward for few tokens (M <= 16): Y = X w_hat^T + s T B^T.
//
// At small batch the layer is bound by reading the 4-bit weights from HBM ("QLoRA --
// Fine-Tuning a 65B Model on One GPU", "Pitfalls": small-batch generation is memory-bound
// and 4 bits leave less to read).  Each weight is decoded once, on chip, from its 4-bit code
// ("QLoRA: Quantize Base Weights to 4-Bit", Section 3) and multiplied on the MFMA units.
//
// Work split: a workgroup owns 16 weight rows and a range of 64-weight blocks; its four
// wavefronts take interleaved blocks.  Lane l handles row n0 + (l & 15) and the 16 weights
// [16g, 16g+16) of each block, g = l >> 4 (an 8-byte code load).  Two MFMA 16x16x32 steps
// cover one block; since all 32 reduction indices of each step lie in that block, its
// constant c1_hat multiplies the 16x16 partial product once, in FP32, before it joins the
// accumulator.  The 16 levels are looked up unscaled (BF16) with byte permutes.
#include "qlora_device.h"
#include "qlora_host.h"

namespace qlora {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

struct BlockIn {
  uint2 code;      // 16 codes of this lane
  uint4 x0, x1;    // X[m, 64b + 16g .. +16]
  uint32_t c8;
  float c2;
};

__device__ __forceinline__ void load_block(const uint8_t* codes_b, const uint8_t* code8,
                                           const float* c2s, const uint16_t* X, int64_t K,
                                           int64_t nrow, bool nok, int64_t mrow, bool mok, int g,
                                           int64_t b, BlockIn& in) {
  const int64_t nb_row = K / kBlock1;
  if (nok) {
    in.code = *reinterpret_cast<const uint2*>(codes_b + nrow * (K / 2) + b * 32 + 8 * g);
    const int64_t blk = nrow * nb_row + b;
    in.c8 = code8[blk];
    in.c2 = c2s[blk >> 8];
  } else {
    in.code = make_uint2(0x88888888u, 0x88888888u);  // the zero level
    in.c8 = 0;
    in.c2 = 0.f;
  }
  if (mok) {
    const uint4* xp = reinterpret_cast<const uint4*>(X + mrow * K + b * 64 + 16 * g);
    in.x0 = xp[0];
    in.x1 = xp[1];
  } else {
    in.x0 = make_uint4(0, 0, 0, 0);
    in.x1 = in.x0;
  }
}

__device__ __forceinline__ void mma_block(const BlockIn& in, const Lut& L, float mu, f32x4_t& acc) {
  uint32_t w0[4], w1[4];
  decode8(in.code.x, L, w0);
  decode8(in.code.y, L, w1);
  const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
  f32x4_t t = mfma16x16x32(as_bf16x8(in.x0), as_bf16x8(w0), z);
  t = mfma16x16x32(as_bf16x8(in.x1), as_bf16x8(w1), t);
  const float c = block_scale(in.c8, in.c2, mu);
  acc[0] = fmaf(c, t[0], acc[0]);
  acc[1] = fmaf(c, t[1], acc[1]);
  acc[2] = fmaf(c, t[2], acc[2]);
  acc[3] = fmaf(c, t[3], acc[3]);
}

// Sum the LoRA-down partials into LDS: sT[m][j] = sum_s Tpart[s][m][j].
__device__ void gather_T(const float* Tpart, int32_t t_splits, int64_t M, int32_t r, float* sT) {
  for (int i = threadIdx.x; i < M * r; i += kThreads) {
    float s = 0.f;
    for (int32_t k = 0; k < t_splits; ++k) s += Tpart[(int64_t)k * M * r + i];
    sT[i] = s;
  }
}

// grid (ceil(N/16), ksplit)
__global__ __launch_bounds__(kThreads) void k_gemv_fwd(
    const uint8_t* __restrict__ codes_b, const uint8_t* __restrict__ code8,
    const float* __restrict__ c2s, const float* __restrict__ mu_p, int64_t N, int64_t K,
    const uint16_t* __restrict__ X, int64_t M, const float* __restrict__ Tpart, int32_t t_splits,
    const uint16_t* __restrict__ B, int32_t r, float s, uint16_t* __restrict__ Y,
    uint16_t* __restrict__ T_save, float* __restrict__ Ypart, int32_t ksplit, Nf4Tables T) {
  __shared__ f32x4_t red[4][64];
  __shared__ float sT[16 * 128];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int64_t nrow = n0 + (lane & 15);
  const int64_t mrow = lane & 15;
  const bool nok = nrow < N, mok = mrow < M;
  const float mu = mu_p[0];
  Lut L;
  load_unscaled_lut(T, L);

  const int64_t nb_row = K / kBlock1;
  const int64_t bps = (nb_row + ksplit - 1) / ksplit;
  const int64_t bbeg = (int64_t)blockIdx.y * bps;
  const int64_t bend = (bbeg + bps < nb_row) ? bbeg + bps : nb_row;

  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  int64_t b = bbeg + wave;
  for (; b + 4 * (kUnroll - 1) < bend; b += 4 * kUnroll) {
    BlockIn in[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) load_block(codes_b, code8, c2s, X, K, nrow, nok, mrow, mok, g, b + 4 * u, in[u]);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) mma_block(in[u], L, mu, acc);
  }
  for (; b < bend; b += 4) {
    BlockIn in;
    load_block(codes_b, code8, c2s, X, K, nrow, nok, mrow, mok, g, b, in);
    mma_block(in, L, mu, acc);
  }
  red[wave][lane] = acc;
  const bool writes_T = T_save && blockIdx.x == 0 && blockIdx.y == 0 && ksplit == 1;
  if (ksplit == 1) gather_T(Tpart, t_splits, M, r, sT);
  __syncthreads();
  if (writes_T) {
    for (int i = threadIdx.x; i < M * r; i += kThreads) T_save[i] = (uint16_t)(pack_bf16x2(sT[i], 0.f) & 0xFFFFu);
  }
  if (wave != 0) return;
  f32x4_t y = red[0][lane];
#pragma unroll
  for (int w = 1; w < 4; ++w) {
    const f32x4_t t = red[w][lane];
    y[0] += t[0]; y[1] += t[1]; y[2] += t[2]; y[3] += t[3];
  }
  // D[m][n]: lane holds rows m = 4g + v, column n = nrow
  if (!nok) return;
  if (ksplit == 1) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t m = 4 * g + v;
      if (m < M) {
        float lo = 0.f;
        for (int32_t j = 0; j < r; ++j) lo = fmaf(sT[m * r + j], bf16lo_to_f32(B[nrow * r + j]), lo);
        const float out = fmaf(s, lo, y[v]);
        Y[m * N + nrow] = (uint16_t)(pack_bf16x2(out, 0.f) & 0xFFFFu);
      }
    }
  } else {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t m = 4 * g + v;
      if (m < M) Ypart[((int64_t)blockIdx.y * M + m) * N + nrow] = y[v];
    }
  }
}

// Y[m][n] = sum_s Ypart[s][m][n] + s * sum_j T[m][j] B[n][j]
__global__ __launch_bounds__(kThreads) void k_gemv_finish(const float* __restrict__ Ypart,
                                                          int32_t ksplit, int64_t M, int64_t N,
                                                          const float* __restrict__ Tpart,
                                                          int32_t t_splits,
                                                          const uint16_t* __restrict__ B, int32_t r,
                                                          float s, uint16_t* __restrict__ Y,
                                                          uint16_t* __restrict__ T_save) {
  __shared__ float sT[16 * 128];
  gather_T(Tpart, t_splits, M, r, sT);
  __syncthreads();
  if (T_save && blockIdx.x == 0) {
    for (int i = threadIdx.x; i < M * r; i += kThreads) T_save[i] = (uint16_t)(pack_bf16x2(sT[i], 0.f) & 0xFFFFu);
  }
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= M * N) return;
  const int64_t m = i / N, n = i % N;
  float y = 0.f;
  for (int32_t k = 0; k < ksplit; ++k) y += Ypart[(int64_t)k * M * N + i];
  float lo = 0.f;
  for (int32_t j = 0; j < r; ++j) lo = fmaf(sT[m * r + j], bf16lo_to_f32(B[n * r + j]), lo);
  Y[i] = (uint16_t)(pack_bf16x2(fmaf(s, lo, y), 0.f) & 0xFFFFu);
}

}  // namespace

hipError_t launch_gemv_fwd(const uint32_t* codes, const uint8_t* code8, const float* c2s,
                           const float* mu, int64_t N, int64_t K, const uint16_t* X, int64_t M,
                           const float* Tpart, int32_t t_splits, const uint16_t* B, int32_t r,
                           float s, uint16_t* Y, uint16_t* T_save, float* Ypart, int32_t ksplit,
                           const Nf4Tables& T, hipStream_t st) {
  dim3 grid((unsigned)((N + 15) / 16), (unsigned)ksplit);
  LaunchTimer t(3, st);
  hipLaunchKernelGGL(k_gemv_fwd, grid, dim3(kThreads), 0, st,
                     reinterpret_cast<const uint8_t*>(codes), code8, c2s, mu, N, K, X, M, Tpart,
                     t_splits, B, r, s, Y, T_save, Ypart, ksplit, T);
  return hipGetLastError();
}

hipError_t launch_gemv_finish(const float* Ypart, int32_t ksplit, int64_t M, int64_t N,
                              const float* Tpart, int32_t t_splits, const uint16_t* B, int32_t r,
                              float s, uint16_t* Y, uint16_t* T_save, hipStream_t st) {
  const int64_t n = M * N;
  hipLaunchKernelGGL(k_gemv_finish, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads),
                     0, st, Ypart, ksplit, M, N, Tpart, t_splits, B, r, s, Y, T_save);
  return hipGetLastError();
}

}  // namespace qlora
