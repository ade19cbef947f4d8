// LoRA side-path kernels.  "QLoRA -- Fine-Tuning a 65B Model on One GPU", "Prerequisite:
// LoRA": A [r, d_in] projects the input down to r dimensions, B [d_out, r] expands it;
// "Where the gradients actually go": only A and B receive gradients.  "QLoRA: Quantize
// Base Weights to 4-Bit", Section 3: the branch is scaled by alpha/r.
//
// rowdot : part[ks][m][j] = sum_{k in split ks} P[m,k] Q[j,k]    (T = X A^T, G = dY B)
//          MFMA 16x16x32 BF16; Q rows are the MFMA A operand, P rows the B operand.
// coldot : part[ms][j][c] = sum_{m in split ms} U[m,j] V[m,c]    (dA = G^T X, dB^T = T^T dY)
//          FP32 FMA over columns c (reduction over tokens m, which are strided in V).
// finish : fixed-order sum of the partials, times the scale, rounded to BF16.
#include "qlora_device.h"
#include "qlora_host.h"

namespace qlora {
namespace {

constexpr int kThreads = 256;
constexpr int kSumU = 16;  // partials loaded together before they are added

// Fixed-order sum of n partials p[0], p[stride], ...; loads of kSumU partials are issued
// before their adds so the sum costs a few memory latencies, not n.
__device__ __forceinline__ float sum_partials(const float* __restrict__ p, int32_t n, int64_t stride) {
  float s = 0.f;
  for (int32_t k0 = 0; k0 < n; k0 += kSumU) {
    float v[kSumU];
#pragma unroll
    for (int u = 0; u < kSumU; ++u) v[u] = (k0 + u < n) ? p[(int64_t)(k0 + u) * stride] : 0.f;
#pragma unroll
    for (int u = 0; u < kSumU; ++u) s += v[u];
  }
  return s;
}

__device__ __forceinline__ uint4 ld16_or_zero(const uint16_t* p, bool ok) {
  return ok ? *reinterpret_cast<const uint4*>(p) : make_uint4(0, 0, 0, 0);
}

// grid (ceil(M/16), ksplit, ceil(R/16)); 4 wavefronts split the WG's k-range in steps of 32.
__global__ __launch_bounds__(kThreads) void k_rowdot(const uint16_t* __restrict__ P,
                                                     const uint16_t* __restrict__ Q, int64_t M,
                                                     int32_t R, int64_t Kd, int64_t kps,
                                                     float* __restrict__ part) {
  __shared__ f32x4_t red[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t m0 = (int64_t)blockIdx.x * 16;
  const int32_t j0 = blockIdx.z * 16;
  const int64_t kbeg = (int64_t)blockIdx.y * kps;
  const int64_t kend = (kbeg + kps < Kd) ? kbeg + kps : Kd;
  const int64_t mrow = m0 + (lane & 15);
  const int32_t jrow = j0 + (lane & 15);
  const int kk = 8 * (lane >> 4);
  const bool mok = mrow < M, jok = jrow < R;
  const uint16_t* pp = P + (mok ? mrow : 0) * Kd + kk;
  const uint16_t* qp = Q + (int64_t)(jok ? jrow : 0) * Kd + kk;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  int64_t k = kbeg + 32 * wave;
  for (; k + 3 * 128 < kend; k += 4 * 128) {
    uint4 pv[4], qv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bool ok = k + 128 * u + kk < kend;
      pv[u] = ld16_or_zero(pp + k + 128 * u, mok && ok);
      qv[u] = ld16_or_zero(qp + k + 128 * u, jok && ok);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc = mfma16x16x32(as_bf16x8(qv[u]), as_bf16x8(pv[u]), acc);
  }
  for (; k < kend; k += 128) {
    const bool ok = k + kk < kend;
    const uint4 pv = ld16_or_zero(pp + k, mok && ok);
    const uint4 qv = ld16_or_zero(qp + k, jok && ok);
    acc = mfma16x16x32(as_bf16x8(qv), as_bf16x8(pv), acc);
  }
  red[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    f32x4_t s = red[0][lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      const f32x4_t t = red[w][lane];
      s[0] += t[0]; s[1] += t[1]; s[2] += t[2]; s[3] += t[3];
    }
    // D[j][m]: lane holds rows j = 4*(lane>>4) + v, column m = lane & 15
    const int64_t m = m0 + (lane & 15);
    if (m < M) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int32_t j = j0 + 4 * (lane >> 4) + v;
        if (j < R) part[((int64_t)blockIdx.y * M + m) * R + j] = s[v];
      }
    }
  }
}

__global__ __launch_bounds__(kThreads) void k_rowdot_finish(const float* __restrict__ part,
                                                            int32_t ksplit, int64_t M, int32_t R,
                                                            float scale, uint16_t* __restrict__ out_s,
                                                            uint16_t* __restrict__ out_u) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= M * R) return;
  const float s = sum_partials(part + i, ksplit, M * R);
  if (out_s) out_s[i] = (uint16_t)(pack_bf16x2(s * scale, 0.f) & 0xFFFFu);
  if (out_u) out_u[i] = (uint16_t)(pack_bf16x2(s, 0.f) & 0xFFFFu);
}

// grid (ceil(C/512), msplit, ceil(R/16)); each thread owns two adjacent columns.
__global__ __launch_bounds__(kThreads) void k_coldot(const uint16_t* __restrict__ U,
                                                     const uint16_t* __restrict__ V, int64_t M,
                                                     int32_t R, int64_t C, int64_t mps,
                                                     float* __restrict__ part) {
  constexpr int kMC = 128;  // token rows staged per pass
  __shared__ float su[kMC][16];
  const int64_t c = (int64_t)blockIdx.x * 512 + 2 * threadIdx.x;
  const int32_t j0 = blockIdx.z * 16;
  const int64_t mbeg = (int64_t)blockIdx.y * mps;
  const int64_t mend = (mbeg + mps < M) ? mbeg + mps : M;
  const bool cok = c < C;
  float a0[16], a1[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) a0[j] = a1[j] = 0.f;
  for (int64_t mc = mbeg; mc < mend; mc += kMC) {
    const int64_t mlen = (mend - mc < kMC) ? mend - mc : kMC;
    __syncthreads();
    for (int t = threadIdx.x; t < kMC * 16; t += kThreads) {
      const int mm = t >> 4, j = t & 15;
      float v = 0.f;
      if (mm < mlen && j0 + j < R) v = bf16lo_to_f32(U[(mc + mm) * R + j0 + j]);
      su[mm][j] = v;
    }
    __syncthreads();
    if (cok) {
      const uint32_t* vp = reinterpret_cast<const uint32_t*>(V + mc * C + c);
      int64_t mm = 0;
      for (; mm + 4 <= mlen; mm += 4) {
        uint32_t w[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) w[u] = vp[(mm + u) * (C / 2)];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float v0 = bf16lo_to_f32(w[u]), v1 = bf16hi_to_f32(w[u]);
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const float uu = su[mm + u][j];
            a0[j] = fmaf(uu, v0, a0[j]);
            a1[j] = fmaf(uu, v1, a1[j]);
          }
        }
      }
      for (; mm < mlen; ++mm) {
        const uint32_t w = vp[mm * (C / 2)];
        const float v0 = bf16lo_to_f32(w), v1 = bf16hi_to_f32(w);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          a0[j] = fmaf(su[mm][j], v0, a0[j]);
          a1[j] = fmaf(su[mm][j], v1, a1[j]);
        }
      }
    }
  }
  if (cok) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j0 + j < R) {
        float* dst = part + ((int64_t)blockIdx.y * R + j0 + j) * C + c;
        *reinterpret_cast<float2*>(dst) = make_float2(a0[j], a1[j]);
      }
    }
  }
}

__global__ __launch_bounds__(kThreads) void k_coldot_finish(const float* __restrict__ part,
                                                            int32_t msplit, int32_t R, int64_t C,
                                                            float scale, int transposed,
                                                            uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;  // i = j*C + c
  if (i >= (int64_t)R * C) return;
  const float s = sum_partials(part + i, msplit, (int64_t)R * C);
  const uint16_t b = (uint16_t)(pack_bf16x2(s * scale, 0.f) & 0xFFFFu);
  if (!transposed) {
    out[i] = b;
  } else {
    const int64_t j = i / C, c = i % C;
    out[c * R + j] = b;
  }
}

__global__ __launch_bounds__(kThreads) void k_transpose_bf16(const uint16_t* __restrict__ in,
                                                             int64_t rows, int64_t cols,
                                                             uint16_t* __restrict__ out) {
  __shared__ uint16_t tile[32][33];
  const int64_t r0 = (int64_t)blockIdx.y * 32, c0 = (int64_t)blockIdx.x * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  for (int y = ty; y < 32; y += 8) {
    const int64_t r = r0 + y, c = c0 + tx;
    tile[y][tx] = (r < rows && c < cols) ? in[r * cols + c] : (uint16_t)0;
  }
  __syncthreads();
  for (int y = ty; y < 32; y += 8) {
    const int64_t c = c0 + y, r = r0 + tx;  // out[c][r]
    if (c < cols && r < rows) out[c * rows + r] = tile[tx][y];
  }
}

}  // namespace

hipError_t launch_rowdot(const uint16_t* P, const uint16_t* Q, int64_t M, int32_t R, int64_t Kd,
                         int32_t ksplit, int64_t k_per_split, float* part, hipStream_t s) {
  dim3 grid((unsigned)((M + 15) / 16), (unsigned)ksplit, (unsigned)((R + 15) / 16));
  LaunchTimer t(6, s);
  hipExtLaunchKernelGGL(k_rowdot, grid, dim3(kThreads), 0, s, t.start, t.stop, 0, P, Q, M, R, Kd, k_per_split, part);
  return hipGetLastError();
}

hipError_t launch_rowdot_finish(const float* part, int32_t ksplit, int64_t M, int32_t R, float scale,
                                uint16_t* out_s, uint16_t* out_u, hipStream_t s) {
  const int64_t n = M * R;
  hipLaunchKernelGGL(k_rowdot_finish, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads),
                     0, s, part, ksplit, M, R, scale, out_s, out_u);
  return hipGetLastError();
}

hipError_t launch_coldot(const uint16_t* U, const uint16_t* V, int64_t M, int32_t R, int64_t C,
                         int32_t msplit, int64_t m_per_split, float* part, hipStream_t s) {
  dim3 grid((unsigned)((C + 511) / 512), (unsigned)msplit, (unsigned)((R + 15) / 16));
  LaunchTimer t(7, s);
  hipExtLaunchKernelGGL(k_coldot, grid, dim3(kThreads), 0, s, t.start, t.stop, 0, U, V, M, R, C, m_per_split, part);
  return hipGetLastError();
}

hipError_t launch_coldot_finish(const float* part, int32_t msplit, int32_t R, int64_t C, float scale,
                                int transposed, uint16_t* out, hipStream_t s) {
  const int64_t n = (int64_t)R * C;
  hipLaunchKernelGGL(k_coldot_finish, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads),
                     0, s, part, msplit, R, C, scale, transposed, out);
  return hipGetLastError();
}

hipError_t launch_transpose_bf16(const uint16_t* in, int64_t rows, int64_t cols, uint16_t* out,
                                 hipStream_t s) {
  dim3 grid((unsigned)((cols + 31) / 32), (unsigned)((rows + 31) / 32));
  hipLaunchKernelGGL(k_transpose_bf16, grid, dim3(kThreads), 0, s, in, rows, cols, out);
  return hipGetLastError();
}

}  // namespace qlora
