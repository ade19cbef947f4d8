// Merge of a trained adapter into the dequantized base, for export as a 16-bit weight:
//   W'[n][k] = bf16( w_hat[n][k] + s * sum_j B[n][j] A[j][k] ),   s = alpha / r
// ("QLoRA: Quantize Base Weights to 4-Bit", "Interview questions": for deployment the base
// is dequantized back to 16 bits and the adapter is folded in, W = W_dequant + (alpha/r) B A;
// "QLoRA -- Fine-Tuning a 65B Model on One GPU", "Pitfalls" and "How it's used in
// practice": the fold happens in 16 bits, and the merged result may be quantized again).
//
// w_hat is decoded exactly as the standalone dequantization does (bf16(fl32(q[code] *
// c1_hat)) through the per-block scaled byte-permute table).  The rank-r product B A is a
// dense contraction and runs on MFMA 32x32x16 BF16 with FP32 accumulation, arranged so the
// accumulator of a lane lines up with the 4-bit codes it decodes:
//   D[i][j] = sum_rho A[rho][k0 + i] B[n0 + j][rho]      (i: weight column, j: weight row)
// Register 4q + v of lane l holds column 8q + 4(l >> 5) + v of row (l & 31): the nibbles
// 4(l >> 5) .. +3 of code word q of that row, so each lane reads one 16-byte run of codes
// per 32x32 tile.  Then v = fl32(w_hat + s * acc) (one fused rounding) and W' = bf16_rne(v).
// A wavefront's 32 x 64 results pass through LDS so they leave as full 128-byte row
// segments with non-temporal stores; the loads are issued in the order they are consumed,
// so the stores of one block overlap the loads of the next.  The kernel moves 2.52 bytes
// per weight (0.52 read, 2 written) and is bound by HBM.
//
// The A operand (reduction index rho strided in memory) is staged per workgroup in LDS,
// rows rho x 256 columns, and read with ds_read_b64_tr_b16: in each 16-lane group, lane i
// receives element i % 4 of the 8 bytes addressed by lanes i/4 + 4t, so if lane j addresses
// row rho0 + j/4, columns c0 + 4 (j % 4) .. +3, lane i receives rows rho0 .. rho0+3 of column
// c0 + i.  The B operand (rho contiguous) is loaded straight into registers once per wave.
#include "qlora_device.h"
#include "qlora_host.h"

namespace qlora {
namespace {

constexpr int kThreads = 256;                // 4 wavefronts
constexpr int kWaves = kThreads / 64;
constexpr int kRowsWG = 32 * kWaves;         // weight rows per workgroup, 32 per wavefront
constexpr int kColsWG = 256;                 // weight columns per workgroup: 8 tiles of 32
constexpr int kTilesK = kColsWG / 32;
constexpr int kPitch = 2 * kColsWG + 64;     // LDS row pitch (bytes): 4 consecutive rows hit
                                             // disjoint bank quarters for the transposing reads
constexpr int kStagePitch = 144;             // output staging: 32 rows x 64 columns per wave

typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

__device__ __forceinline__ f32x16_t mfma32(const bf16x8_t& a, const bf16x8_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// A operand of one 32x32x16 MFMA: lane l receives rows 8 (l >> 5) .. +7 of column (l & 31)
// of the LDS tile starting at `tile` (16 rows of the rank index, kPitch bytes apart).
__device__ __forceinline__ bf16x8_t tr32_operand(const char* tile, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const char* p0 = tile + (8 * (g >> 1) + (j >> 2)) * kPitch + 2 * (16 * (g & 1) + 4 * (j & 3));
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p0));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p0 + 4 * kPitch));
  bf16x8_t r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}

// Four BF16 values of one code word: elements 4h .. 4h+3 (nibble half h) as two BF16 pairs.
__device__ __forceinline__ void decode4(uint32_t u, int h, const Lut& L, uint32_t& p01, uint32_t& p23) {
  const uint32_t idx = (u >> (4 * h)) & 0x0F0F0F0Fu;
  const uint32_t idx8 = idx ^ 0x08080808u;
  const uint32_t m = nib_mask(idx);
  const uint32_t lo = lut16(idx, idx8, m, L.lo[0], L.lo[1], L.lo[2], L.lo[3]);
  const uint32_t hi = lut16(idx, idx8, m, L.hi[0], L.hi[1], L.hi[2], L.hi[3]);
  p01 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
  p23 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
}

// grid: (ceil(K / 256), ceil(N / 128)).  RC = ceil(r / 16) rank chunks.
template <int RC, int DQ>
__global__ __launch_bounds__(kThreads) void k_merge(const uint32_t* __restrict__ codes,
                                                    const uint8_t* __restrict__ code8,
                                                    const float* __restrict__ c2s,
                                                    const float* __restrict__ mu,
                                                    const uint16_t* __restrict__ A,
                                                    const uint16_t* __restrict__ B, int64_t N, int64_t K,
                                                    int32_t r, float s, uint16_t* __restrict__ out,
                                                    Nf4Tables T) {
  __shared__ __attribute__((aligned(16))) char sa[16 * RC * kPitch];
  __shared__ __attribute__((aligned(16))) char so[kWaves * 32 * kStagePitch];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, h32 = lane >> 5;
  const int64_t k0 = (int64_t)blockIdx.x * kColsWG;
  const int64_t n = (int64_t)blockIdx.y * kRowsWG + 32 * wave + l32;
  const bool row_ok = n < N;
  const int64_t nb_row = K / kBlock1, nb = N * nb_row;

  // Loads are issued in the order they are consumed -- A (staged before the barrier), B,
  // the block constants, then the code words tile by tile -- so each wait below covers only
  // what its step needs and the stores of one block overlap the loads of the next.
  constexpr int kStage = 16 * RC * (kColsWG / 8);  // 16-byte pieces of the A tile
  constexpr int kStageIt = (kStage + kThreads - 1) / kThreads;
  const rsrc_t ra = make_rsrc(A, (int64_t)r * K * 2);
  uint4 av[kStageIt];
#pragma unroll
  for (int it = 0; it < kStageIt; ++it) {
    const int idx = threadIdx.x + kThreads * it;
    const int row = idx / (kColsWG / 8), ch = idx % (kColsWG / 8);
    const int64_t k = k0 + 8 * ch;
    av[it] = bload16(ra, (idx < kStage && row < r && k < K) ? (uint32_t)(((int64_t)row * K + k) * 2) : kOOB);
  }

  // B operand: row n, rank indices 16 c + 8 h32 .. +7
  const rsrc_t rb = make_rsrc(B, N * r * 2);
  bf16x8_t bop[RC];
#pragma unroll
  for (int c = 0; c < RC; ++c) {
    const int rho = 16 * c + 8 * h32;
    if ((r & 7) == 0) {
      bop[c] = as_bf16x8(bload16(rb, (row_ok && rho < r) ? (uint32_t)((n * r + rho) * 2) : kOOB));
    } else {
      uint32_t e[8];
#pragma unroll
      for (int q = 0; q < 8; ++q)
        e[q] = __builtin_amdgcn_raw_buffer_load_b16(rb, (row_ok && rho + q < r) ? (int)((n * r + rho + q) * 2) : (int)kOOB,
                                                     0, 0);
      const uint4 v = make_uint4((e[0] & 0xFFFFu) | (e[1] << 16), (e[2] & 0xFFFFu) | (e[3] << 16),
                                 (e[4] & 0xFFFFu) | (e[5] << 16), (e[6] & 0xFFFFu) | (e[7] << 16));
      bop[c] = as_bf16x8(v);
    }
  }

  // block constants of the blocks of 64 columns
  const rsrc_t r8 = make_rsrc(code8, DQ == kDqNone ? 4 * nb : nb);
  const rsrc_t r2 = make_rsrc(c2s, 4 * ((nb + kBlock2 - 1) / kBlock2));
  uint32_t c8[kTilesK / 2];
  float g2[kTilesK / 2];
#pragma unroll
  for (int b = 0; b < kTilesK / 2; ++b) {
    const bool ok = row_ok && k0 + 64 * b < K;
    const int64_t blk = n * nb_row + k0 / kBlock1 + b;
    if (DQ == kDqNone) {  // the FP32 constant itself
      c8[b] = bload4(r8, ok ? (uint32_t)(4 * blk) : kOOB);
      g2[b] = 0.f;
    } else {
      c8[b] = bload1(r8, ok ? (uint32_t)blk : kOOB);
      g2[b] = __uint_as_float(bload4(r2, ok ? (uint32_t)(4 * ((uint64_t)blk >> 8)) : kOOB));
    }
  }
  const float mu0 = DQ == kDqNone ? 0.f : mu[0];

  // this lane's code words: tile i holds columns k0 + 32 i .. +31 (16 bytes of codes)
  const rsrc_t rc = make_rsrc(codes, N * K / 2);
  uint4 cw[kTilesK];
#pragma unroll
  for (int i = 0; i < kTilesK; ++i)
    cw[i] = bload16(rc, (row_ok && k0 + 32 * i < K) ? (uint32_t)((uint64_t)(n * K + k0 + 32 * i) >> 1) : kOOB);

  // A[0 .. 16 RC)[k0 .. k0 + kColsWG) into LDS (zeros beyond r and K); the barrier waits for
  // LDS traffic only, not for the loads still in flight
#pragma unroll
  for (int it = 0; it < kStageIt; ++it) {
    const int idx = threadIdx.x + kThreads * it;
    if (idx < kStage) *reinterpret_cast<uint4*>(sa + (idx / (kColsWG / 8)) * kPitch + 16 * (idx % (kColsWG / 8))) = av[it];
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("s_barrier" ::: "memory");

  char* stg = so + wave * 32 * kStagePitch;
#pragma unroll
  for (int bb = 0; bb < kTilesK / 2; ++bb) {
    // uniform per workgroup (K is a multiple of 64); rows past N still run the MFMAs and the
    // transposing reads, which gather across lanes, and only skip the stores
    if (k0 + 64 * bb >= K) break;
    Lut L;
    build_scaled_lut(T, block_scale_fmt<DQ>(c8[bb], g2[bb], mu0), L);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int i = 2 * bb + half;
      f32x16_t acc;
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[v] = 0.f;
#pragma unroll
      for (int c = 0; c < RC; ++c) acc = mfma32(tr32_operand(sa + 16 * c * kPitch + 64 * i, lane), bop[c], acc);
      const uint32_t words[4] = {cw[i].x, cw[i].y, cw[i].z, cw[i].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t p01, p23;
        decode4(words[q], h32, L, p01, p23);
        const float v0 = fmaf(s, acc[4 * q + 0], bf16lo_to_f32(p01));
        const float v1 = fmaf(s, acc[4 * q + 1], bf16hi_to_f32(p01));
        const float v2 = fmaf(s, acc[4 * q + 2], bf16lo_to_f32(p23));
        const float v3 = fmaf(s, acc[4 * q + 3], bf16hi_to_f32(p23));
        *reinterpret_cast<uint2*>(stg + l32 * kStagePitch + 2 * (32 * half + 8 * q + 4 * h32)) =
            make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
      }
    }
    // the wavefront's 32 x 64 block goes out as 8 full 128-byte row segments per store,
    // bypassing the caches on the way (the export is not read back here)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int row = 8 * t + (lane >> 3), ch = lane & 7;
      const uint4 v = *reinterpret_cast<const uint4*>(stg + row * kStagePitch + 16 * ch);
      const int64_t nr = (int64_t)blockIdx.y * kRowsWG + 32 * wave + row;
      if (nr < N)
        __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w},
                                    reinterpret_cast<u32x4_t*>(out + nr * K + k0 + 64 * bb + 8 * ch));
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_wave_barrier();
  }
}

template <int RC>
hipError_t launch_rc(dim3 grid, const LaunchTimer& t, hipStream_t st, const uint32_t* codes, const uint8_t* code8,
                     const float* c2s, const float* mu, const uint16_t* A, const uint16_t* B, int64_t N, int64_t K,
                     int32_t r, float s, uint16_t* out, const Nf4Tables& T, int dq) {
  auto go = [&](auto kern) {
    hipExtLaunchKernelGGL(kern, grid, dim3(kThreads), 0, st, t.start, t.stop, 0, codes, code8, c2s, mu, A, B, N, K, r, s,
                          out, T);
  };
  if (dq == kDqE5M2) go(k_merge<RC, kDqE5M2>);
  else if (dq == kDqInt8) go(k_merge<RC, kDqInt8>);
  else if (dq == kDqNone) go(k_merge<RC, kDqNone>);
  else go(k_merge<RC, kDqE4M3>);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(const uint32_t* codes, const uint8_t* code8, const float* c2s, const float* mu,
                        const uint16_t* A, const uint16_t* B, int64_t N, int64_t K, int32_t r, float s,
                        uint16_t* out, const Nf4Tables& T, int dq, hipStream_t st) {
  const dim3 grid((unsigned)((K + kColsWG - 1) / kColsWG), (unsigned)((N + kRowsWG - 1) / kRowsWG));
  LaunchTimer t(9, st);
  switch ((r + 15) / 16) {
    case 1: return launch_rc<1>(grid, t, st, codes, code8, c2s, mu, A, B, N, K, r, s, out, T, dq);
    case 2: return launch_rc<2>(grid, t, st, codes, code8, c2s, mu, A, B, N, K, r, s, out, T, dq);
    case 3: return launch_rc<3>(grid, t, st, codes, code8, c2s, mu, A, B, N, K, r, s, out, T, dq);
    case 4: return launch_rc<4>(grid, t, st, codes, code8, c2s, mu, A, B, N, K, r, s, out, T, dq);
    case 5: return launch_rc<5>(grid, t, st, codes, code8, c2s, mu, A, B, N, K, r, s, out, T, dq);
    case 6: return launch_rc<6>(grid, t, st, codes, code8, c2s, mu, A, B, N, K, r, s, out, T, dq);
    case 7: return launch_rc<7>(grid, t, st, codes, code8, c2s, mu, A, B, N, K, r, s, out, T, dq);
    case 8: return launch_rc<8>(grid, t, st, codes, code8, c2s, mu, A, B, N, K, r, s, out, T, dq);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qlora
