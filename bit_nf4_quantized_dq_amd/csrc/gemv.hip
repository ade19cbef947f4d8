// Weight-streaming forward for few tokens (M <= 16): Y = X w_hat^T + s (X A^T) B^T, one launch.
//
// At small batch the layer is bound by reading the 4-bit weights from HBM ("QLoRA --
// Fine-Tuning a 65B Model on One GPU", "Pitfalls": small-batch generation is memory-bound
// and 4 bits leave less to read).  Each weight is decoded once, on chip, from its 4-bit code
// ("QLoRA: Quantize Base Weights to 4-Bit", Section 3) and multiplied on the MFMA units.
//
// Work split.  A workgroup owns 128 weight rows (8 wavefronts x one MFMA column tile of 16
// rows) and one of `ksplit` ranges of 64-weight blocks, walked in chunks of kChunk blocks.
// Per chunk, every thread first issues all of its global loads (part of one weight row's
// codes and block constants, a slice of X) into registers, then writes them to LDS; the MFMA
// loop then reads LDS, while the next chunk's loads are in flight.  Lane l handles rows 16t + (l & 15) and, in each block, the 16 weights
// [16g, 16g+16), g = l >> 4.  Two MFMA 16x16x32 steps cover a block; all 32 reduction
// indices of each step lie in that block, so its constant c1_hat multiplies the 16x16
// partial product once, in FP32, before it joins the accumulator.  The 16 levels are looked
// up unscaled (BF16) with byte permutes.  The block loop over a staged chunk is unrolled
// without bounds tests: blocks past the end of the slice hold zero activations (and finite
// decoded weights), so they add exact zeros.
//
// Adapter.  T = X A^T is linear in the reduction range, so each workgroup forms the part of
// T over its own k-range (its wavefronts take interleaved blocks), applies B to it for its
// 128 rows, and adds that to its partial output.
//
// Split-K reduction.  With ksplit > 1 each workgroup writes an FP32 partial; the last
// workgroup of a row group to finish (a device-scope arrival counter, one per row group, in
// the caller's workspace; that workgroup resets it to zero) sums the partials in a fixed
// order and writes BF16 Y (and T for the backward).  Calls that share a workspace must not
// overlap; calls with separate workspaces may.  The partials travel through memory with system-scope (cache-bypassing) stores and loads:
// the writer waits for its stores to complete before advancing the counter, so the reader
// needs no cache write-back fence.
#include "qlora_device.h"
#include "qlora_host.h"

namespace qlora {

namespace {

// Workgroup barrier that waits for this wavefront's LDS accesses only (lgkmcnt), so global
// loads in flight stay in flight across it.  Every barrier here orders LDS traffic between
// the wavefronts; none orders global memory.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("s_barrier" ::: "memory");
}

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kTiles = 1;               // column tiles (16 rows) per wavefront
constexpr int kRows = kWaves * 16 * kTiles;  // rows per workgroup
constexpr int kChunk = 8;               // blocks staged per pass (all loads of a pass in flight at once)
constexpr int kXItems = 16 * kChunk * 8 / kThreads;  // 16-byte pieces of X staged per thread per pass
constexpr int kStageBlocks = kChunk * kRows / kThreads;  // blocks of one row staged per thread
constexpr int32_t kMaxSplit = 65536;
constexpr int kSumU = 16;               // partials loaded together in the split-K sum

struct GemvArgs {
  const uint8_t* codes;
  const uint8_t* code8;
  const float* c2s;
  const float* mu;
  int64_t N, K;
  const uint16_t* X;
  int64_t M;
  const uint16_t* A;
  const uint16_t* B;
  int32_t r;
  float s;
  uint16_t* Y;
  uint16_t* T_save;
  float* part;   // [ksplit][M][N]
  float* tpart;  // [ksplit][M][r]
  unsigned int* counters;  // [row groups], zero between calls
  int32_t ksplit;
  int32_t nbs;   // blocks per split
};

__device__ __forceinline__ void publish(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ float sum_published(const float* p, int32_t n, int64_t stride) {
  float s = 0.f;
  for (int32_t k0 = 0; k0 < n; k0 += kSumU) {
    float v[kSumU];
#pragma unroll
    for (int u = 0; u < kSumU; ++u)
      v[u] = (k0 + u < n) ? __hip_atomic_load(p + (int64_t)(k0 + u) * stride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) : 0.f;
#pragma unroll
    for (int u = 0; u < kSumU; ++u) s += v[u];
  }
  return s;
}

// Token and row of output i (< M nrows <= 16 kRows) of a row group with nrows rows: 32-bit,
// and shifts for a whole group (a 64-bit division is a long instruction sequence, and these
// sit in the launch's critical tail).
__device__ __forceinline__ void split_out(int i, int nrows, int& m, int& nn) {
  m = nrows == kRows ? (int)((unsigned)i / (unsigned)kRows) : (int)((unsigned)i / (unsigned)nrows);
  nn = i - m * nrows;
}

// The same fixed-order sum for up to kSumOut outputs of one thread at once (output i0 + o
// kThreads, o < kSumOut, of `total`; output i is Y[i / nrows][row0 + i % nrows] of a row-major
// [M][N] partial), all of their loads issued before any is summed.
constexpr int kSumOut = 4;
constexpr int kSumOutU = 8;  // partials per output loaded together there
__device__ __forceinline__ void sum_published_n(const float* part, int64_t i0, int64_t total, int64_t nrows,
                                                int64_t row0, int64_t N, int32_t n, int64_t stride,
                                                float (&sum)[kSumOut]) {
#pragma unroll
  for (int o = 0; o < kSumOut; ++o) sum[o] = 0.f;
  for (int32_t k0 = 0; k0 < n; k0 += kSumOutU) {
    float v[kSumOut][kSumOutU];
#pragma unroll
    for (int o = 0; o < kSumOut; ++o) {
      const int64_t i = i0 + (int64_t)o * kThreads;
      int m, nn;
      split_out((int)i, (int)nrows, m, nn);
      const float* p = part + (int64_t)m * N + row0 + nn;
#pragma unroll
      for (int u = 0; u < kSumOutU; ++u)
        v[o][u] = (i < total && k0 + u < n)
                      ? __hip_atomic_load(p + (int64_t)(k0 + u) * stride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM)
                      : 0.f;
    }
#pragma unroll
    for (int o = 0; o < kSumOut; ++o)
#pragma unroll
      for (int u = 0; u < kSumOutU; ++u) sum[o] += v[o][u];
  }
}

// Rows are padded so the 16 lanes that read 16 consecutive rows hit distinct LDS banks.
struct Stage {
  uint2 codes[kRows][kChunk * 4 + 1];  // row, (block, 8-byte part g) at 4 * block + g
  float scale[kRows][kChunk + 1];
  uint4 x[16][kChunk * 8 + 1];         // X[m][64 b + 8 c .. +8] at 8 * b + c
};
constexpr int kRStage = 32;       // adapter ranks whose B rows are prefetched into LDS

// Registers holding one chunk's global loads between issue and the LDS write.
struct ChunkRegs {
  uint4 cv[kStageBlocks][2];
  uint32_t c8[kStageBlocks], c2[kStageBlocks];
  uint4 xv[kXItems];
};

// ONE: the workgroup's range is exactly one full chunk (e.g. 4096x4096).  Then the adapter
// part runs first, while the codes are still in flight: X, the A pieces and the B rows are
// issued before the codes, so waiting for them (loads complete in issue order) does not wait
// for the codes, and T, its cross-wavefront sum and the up-projection overlap the code
// transfer.  The chunk loop below is the general path.
template <int RT, bool ONE>  // RT: 16-wide tiles of the adapter rank, r <= 16 * RT
__global__ __launch_bounds__(kThreads) void k_gemv_fused(GemvArgs a, Nf4Tables T) {
  __shared__ Stage S;
  __shared__ f32x4_t sred[kWaves][RT][64];
  __shared__ float sT[16][16 * RT + 1];
  __shared__ unsigned int s_last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int64_t N = a.N, K = a.K, M = a.M;
  const int64_t nb_row = K / kBlock1;
  const int64_t grp = blockIdx.x;
  const int ks = blockIdx.y;
  const int64_t b0 = (int64_t)ks * a.nbs;
  const int64_t b1 = (b0 + a.nbs < nb_row) ? b0 + a.nbs : nb_row;
  const float mu = a.mu[0];
  const int64_t row0 = grp * kRows;

  const rsrc_t rc = make_rsrc(a.codes, N * (K / 2));
  const rsrc_t r8 = make_rsrc(a.code8, N * nb_row);
  const rsrc_t r2 = make_rsrc(a.c2s, ((N * nb_row + 255) / 256) * 4);
  const rsrc_t rx = make_rsrc(a.X, M * K * 2);
  const rsrc_t ra = make_rsrc(a.A, (int64_t)a.r * K * 2);
  Lut L;
  load_unscaled_lut(T, L);

  f32x4_t acc[kTiles];
  f32x4_t tacc[RT];
#pragma unroll
  for (int t = 0; t < kTiles; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < RT; ++j) tacc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const f32x4_t z = {0.f, 0.f, 0.f, 0.f};

  // staging roles: thread tid stages blocks [sb0, sb0 + kStageBlocks) of the chunk for weight
  // row row0 + srow and, for X, row tid >> 4 at the 16-byte column tid & 15 of each pair of
  // blocks
  const int srow = tid % kRows, sb0 = (tid / kRows) * kStageBlocks;
  const uint32_t my_code_off = (uint32_t)((row0 + srow) * (K / 2));
  const uint32_t my_blk = (uint32_t)((row0 + srow) * nb_row);

  // B rows of this workgroup for the adapter up-projection, prefetched with the first chunk
  __shared__ uint4 sB[kRows][kRStage / 8];
  uint4 bpre[kRStage / 8];
  if (!ONE) {
    const rsrc_t rb = make_rsrc(a.B, N * a.r * 2);
    const bool pre = (a.r % 8) == 0 && a.r <= kRStage;
#pragma unroll
    for (int q = 0; q < kRStage / 8; ++q)
      bpre[q] = bload16(rb, (pre && 8 * q < a.r && tid < kRows) ? (uint32_t)(((row0 + tid) * a.r + 8 * q) * 2) : kOOB);
  }

  auto issue = [&](int64_t c0, ChunkRegs& R) {
    const int nb = (b1 - c0 < kChunk) ? (int)(b1 - c0) : kChunk;
#pragma unroll
    for (int v = 0; v < kStageBlocks; ++v) {
      const int u = sb0 + v;
      const bool ok = u < nb;
      const uint32_t off = my_code_off + (uint32_t)((c0 + u) * 32);
      R.cv[v][0] = bload16(rc, ok ? off : kOOB);
      R.cv[v][1] = bload16(rc, ok ? off + 16 : kOOB);
      const uint32_t bi = my_blk + (uint32_t)(c0 + u);
      R.c8[v] = bload1(r8, ok ? bi : kOOB);
      R.c2[v] = bload4(r2, ok ? (bi >> 8) * 4 : kOOB);
    }
#pragma unroll
    for (int p = 0; p < kXItems; ++p) {  // item i: X row i / (8 kChunk), 16-byte piece i % (8 kChunk)
      const int i = tid + kThreads * p, xm = i / (8 * kChunk), col = i % (8 * kChunk);
      const int64_t k = 64 * (c0 + col / 8) + 8 * (col % 8);
      const bool ok = c0 + col / 8 < b1;
      R.xv[p] = bload16(rx, ok ? (uint32_t)((xm * K + k) * 2) : kOOB);
    }
  };
  auto stage = [&](const ChunkRegs& R) {
#pragma unroll
    for (int v = 0; v < kStageBlocks; ++v) {
      const int u = sb0 + v;
      S.codes[srow][4 * u + 0] = make_uint2(R.cv[v][0].x, R.cv[v][0].y);
      S.codes[srow][4 * u + 1] = make_uint2(R.cv[v][0].z, R.cv[v][0].w);
      S.codes[srow][4 * u + 2] = make_uint2(R.cv[v][1].x, R.cv[v][1].y);
      S.codes[srow][4 * u + 3] = make_uint2(R.cv[v][1].z, R.cv[v][1].w);
      S.scale[srow][u] = block_scale(R.c8[v], __uint_as_float(R.c2[v]), mu);
    }
#pragma unroll
    for (int p = 0; p < kXItems; ++p) {
      const int i = tid + kThreads * p;
      S.x[i / (8 * kChunk)][i % (8 * kChunk)] = R.xv[p];
    }
  };

  if constexpr (ONE) {
    static_assert(kChunk == kWaves && kTiles == 1, "one adapter block and one row tile per wavefront");
    const int nb = (int)(b1 - b0);
    const int u = wave;
    // X pieces of the chunk, then this wavefront's A pieces, then the B rows, then the codes
    uint4 xv[kXItems];
#pragma unroll
    for (int p = 0; p < kXItems; ++p) {
      const int i = tid + kThreads * p, xm = i / (8 * kChunk), col = i % (8 * kChunk);
      const int64_t k = 64 * (b0 + col / 8) + 8 * (col % 8);
      xv[p] = bload16(rx, b0 + col / 8 < b1 ? (uint32_t)((xm * K + k) * 2) : kOOB);
    }
    uint4 av[RT][2];
#pragma unroll
    for (int j = 0; j < RT; ++j) {
      const bool ok = u < nb && 16 * j + l16 < a.r;
      const uint32_t ao = (uint32_t)((((int64_t)(16 * j + l16)) * K + 64 * (b0 + u) + 16 * g) * 2);
      av[j][0] = bload16(ra, ok ? ao : kOOB);
      av[j][1] = bload16(ra, ok ? ao + 16 : kOOB);
    }
    {
      const rsrc_t rb = make_rsrc(a.B, N * a.r * 2);
      const bool pre = (a.r % 8) == 0 && a.r <= kRStage;
#pragma unroll
      for (int q = 0; q < kRStage / 8; ++q)
        bpre[q] = bload16(rb, (pre && 8 * q < a.r && tid < kRows) ? (uint32_t)(((row0 + tid) * a.r + 8 * q) * 2) : kOOB);
    }
    uint4 cv[kStageBlocks][2];
    uint32_t c8[kStageBlocks], c2[kStageBlocks];
#pragma unroll
    for (int v = 0; v < kStageBlocks; ++v) {
      const int ub = sb0 + v;
      const bool ok = ub < nb;
      const uint32_t off = my_code_off + (uint32_t)((b0 + ub) * 32);
      cv[v][0] = bload16(rc, ok ? off : kOOB);
      cv[v][1] = bload16(rc, ok ? off + 16 : kOOB);
      const uint32_t bi = my_blk + (uint32_t)(b0 + ub);
      c8[v] = bload1(r8, ok ? bi : kOOB);
      c2[v] = bload4(r2, ok ? (bi >> 8) * 4 : kOOB);
    }
    // adapter part while the codes travel
#pragma unroll
    for (int p = 0; p < kXItems; ++p) {
      const int i = tid + kThreads * p;
      S.x[i / (8 * kChunk)][i % (8 * kChunk)] = xv[p];
    }
    if (tid < kRows) {
#pragma unroll
      for (int q = 0; q < kRStage / 8; ++q) sB[tid][q] = bpre[q];
    }
    lds_barrier();
    if (u < nb) {
      const bf16x8_t xa = as_bf16x8(S.x[l16][8 * u + 2 * g]);
      const bf16x8_t xb = as_bf16x8(S.x[l16][8 * u + 2 * g + 1]);
#pragma unroll
      for (int j = 0; j < RT; ++j) {
        tacc[j] = mfma16x16x32(xa, as_bf16x8(av[j][0]), tacc[j]);
        tacc[j] = mfma16x16x32(xb, as_bf16x8(av[j][1]), tacc[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < RT; ++j) sred[wave][j][lane] = tacc[j];
    lds_barrier();
    for (int i = tid; i < 16 * 16 * RT; i += kThreads) {
      const int j16 = i / 256, rem = i % 256, ln = rem / 4, v = rem % 4;  // D[m = 4*(ln>>4)+v][j = ln & 15]
      float s = sred[0][j16][ln][v];
      for (int w = 1; w < kWaves; ++w) s += sred[w][j16][ln][v];
      sT[4 * (ln >> 4) + v][16 * j16 + (ln & 15)] = s;
    }
    lds_barrier();
    for (int32_t j0 = 0; j0 < a.r; j0 += 32) {  // r <= 32 here, so B comes from LDS or element loads
      const int32_t jj = j0 + 8 * g;
      uint32_t tv[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float lo = (jj + 2 * q < a.r) ? a.s * sT[l16][jj + 2 * q] : 0.f;
        const float hi = (jj + 2 * q + 1 < a.r) ? a.s * sT[l16][jj + 2 * q + 1] : 0.f;
        tv[q] = pack_bf16x2(lo, hi);
      }
      const int rl = wave * 16 + l16;
      uint4 bw;
      if ((a.r % 8) == 0) {
        bw = (jj < a.r) ? sB[rl][jj / 8] : make_uint4(0, 0, 0, 0);
      } else {
        const rsrc_t rb = make_rsrc(a.B, N * a.r * 2);
        const int64_t n = row0 + rl;
        uint32_t e[8];
#pragma unroll
        for (int q = 0; q < 8; ++q)
          e[q] = __builtin_amdgcn_raw_buffer_load_b16(rb, (jj + q < a.r) ? (int)((n * a.r + jj + q) * 2) : (int)kOOB, 0, 0);
        bw = make_uint4((e[0] & 0xFFFFu) | (e[1] << 16), (e[2] & 0xFFFFu) | (e[3] << 16),
                        (e[4] & 0xFFFFu) | (e[5] << 16), (e[6] & 0xFFFFu) | (e[7] << 16));
      }
      acc[0] = mfma16x16x32(as_bf16x8(tv), as_bf16x8(bw), acc[0]);
    }
    // the codes: stage, then the chunk's MFMAs on top of the adapter term
#pragma unroll
    for (int v = 0; v < kStageBlocks; ++v) {
      const int ub = sb0 + v;
      S.codes[srow][4 * ub + 0] = make_uint2(cv[v][0].x, cv[v][0].y);
      S.codes[srow][4 * ub + 1] = make_uint2(cv[v][0].z, cv[v][0].w);
      S.codes[srow][4 * ub + 2] = make_uint2(cv[v][1].x, cv[v][1].y);
      S.codes[srow][4 * ub + 3] = make_uint2(cv[v][1].z, cv[v][1].w);
      S.scale[srow][ub] = block_scale(c8[v], __uint_as_float(c2[v]), mu);
    }
    lds_barrier();
#pragma unroll
    for (int ub = 0; ub < kChunk; ++ub) {
      const bf16x8_t xa = as_bf16x8(S.x[l16][8 * ub + 2 * g]);
      const bf16x8_t xb = as_bf16x8(S.x[l16][8 * ub + 2 * g + 1]);
      const int row = wave * 16 + l16;
      const uint2 cw = S.codes[row][4 * ub + g];
      uint32_t w0[4], w1[4];
      decode8(cw.x, L, w0);
      decode8(cw.y, L, w1);
      f32x4_t p = mfma16x16x32(xa, as_bf16x8(w0), z);
      p = mfma16x16x32(xb, as_bf16x8(w1), p);
      const float c = S.scale[row][ub];
      acc[0][0] = fmaf(c, p[0], acc[0][0]);
      acc[0][1] = fmaf(c, p[1], acc[0][1]);
      acc[0][2] = fmaf(c, p[2], acc[0][2]);
      acc[0][3] = fmaf(c, p[3], acc[0][3]);
    }
  } else {
    ChunkRegs R;
    issue(b0, R);
    if (tid < kRows) {
#pragma unroll
      for (int q = 0; q < kRStage / 8; ++q) sB[tid][q] = bpre[q];
    }
    for (int64_t c0 = b0; c0 < b1; c0 += kChunk) {
      const int nb = (b1 - c0 < kChunk) ? (int)(b1 - c0) : kChunk;
      // adapter down-projection inputs of this chunk: wavefront w takes blocks u = w (mod kWaves);
      // for r <= 32 they are issued here, with the chunk, for larger r when the block comes up
      constexpr int kTA = RT <= 2 ? (kChunk + kWaves - 1) / kWaves : 1;
      uint4 av[kTA][RT][2];
      auto load_a = [&](int u, uint4 (&dst)[RT][2]) {
#pragma unroll
        for (int j = 0; j < RT; ++j) {
          const bool ok = u < nb && 16 * j + l16 < a.r;
          const uint32_t ao = (uint32_t)((((int64_t)(16 * j + l16)) * K + 64 * (c0 + u) + 16 * g) * 2);
          dst[j][0] = bload16(ra, ok ? ao : kOOB);
          dst[j][1] = bload16(ra, ok ? ao + 16 : kOOB);
        }
      };
      if (RT <= 2) {
#pragma unroll
        for (int q = 0; q < kTA; ++q) load_a(kWaves * q + wave, av[q]);
      }
      lds_barrier();  // the previous chunk's LDS reads are done
      stage(R);
      lds_barrier();
      if (c0 + kChunk < b1) issue(c0 + kChunk, R);  // next chunk in flight during this one's math

      // ---- adapter down-projection share of this wavefront: blocks u = wave (mod kWaves)
      if (RT <= 2) {
#pragma unroll
        for (int q = 0; q < kTA; ++q) {
          const int u = kWaves * q + wave;
          if (u < nb) {
            const bf16x8_t xa = as_bf16x8(S.x[l16][8 * u + 2 * g]);
            const bf16x8_t xb = as_bf16x8(S.x[l16][8 * u + 2 * g + 1]);
#pragma unroll
            for (int j = 0; j < RT; ++j) {
              tacc[j] = mfma16x16x32(xa, as_bf16x8(av[q][j][0]), tacc[j]);
              tacc[j] = mfma16x16x32(xb, as_bf16x8(av[q][j][1]), tacc[j]);
            }
          }
        }
      } else {
        for (int u = wave; u < nb; u += kWaves) {
          load_a(u, av[0]);
          const bf16x8_t xa = as_bf16x8(S.x[l16][8 * u + 2 * g]);
          const bf16x8_t xb = as_bf16x8(S.x[l16][8 * u + 2 * g + 1]);
#pragma unroll
          for (int j = 0; j < RT; ++j) {
            tacc[j] = mfma16x16x32(xa, as_bf16x8(av[0][j][0]), tacc[j]);
            tacc[j] = mfma16x16x32(xb, as_bf16x8(av[0][j][1]), tacc[j]);
          }
        }
      }
      // ---- MFMA over the staged chunk
      // blocks past the slice (u >= nb) hold zero activations, so they add exact zeros
#pragma unroll
      for (int u = 0; u < kChunk; ++u) {
        const bf16x8_t xa = as_bf16x8(S.x[l16][8 * u + 2 * g]);
        const bf16x8_t xb = as_bf16x8(S.x[l16][8 * u + 2 * g + 1]);
#pragma unroll
        for (int t = 0; t < kTiles; ++t) {
          const int row = wave * 16 * kTiles + 16 * t + l16;
          const uint2 cw = S.codes[row][4 * u + g];
          uint32_t w0[4], w1[4];
          decode8(cw.x, L, w0);
          decode8(cw.y, L, w1);
          f32x4_t p = mfma16x16x32(xa, as_bf16x8(w0), z);
          p = mfma16x16x32(xb, as_bf16x8(w1), p);
          const float c = S.scale[row][u];
          acc[t][0] = fmaf(c, p[0], acc[t][0]);
          acc[t][1] = fmaf(c, p[1], acc[t][1]);
          acc[t][2] = fmaf(c, p[2], acc[t][2]);
          acc[t][3] = fmaf(c, p[3], acc[t][3]);
        }
      }
    }

    // ---- T over this k-range: sum the wavefronts' shares -> sT[m][j]
#pragma unroll
    for (int j = 0; j < RT; ++j) sred[wave][j][lane] = tacc[j];
    lds_barrier();
    for (int i = tid; i < 16 * 16 * RT; i += kThreads) {
      const int j16 = i / 256, rem = i % 256, ln = rem / 4, v = rem % 4;  // D[m = 4*(ln>>4)+v][j = ln & 15]
      float s = sred[0][j16][ln][v];
      for (int w = 1; w < kWaves; ++w) s += sred[w][j16][ln][v];
      sT[4 * (ln >> 4) + v][16 * j16 + (ln & 15)] = s;
    }
    lds_barrier();

    // ---- adapter up-projection of this partial T: acc[t][m][n] += s * sum_j T[m][j] B[n][j]
    const bool b_staged = (a.r % 8) == 0 && a.r <= kRStage;
    const rsrc_t rb = make_rsrc(a.B, N * a.r * 2);
    for (int32_t j0 = 0; j0 < a.r; j0 += 32) {
      const int32_t jj = j0 + 8 * g;
      uint32_t tv[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float lo = (jj + 2 * q < a.r) ? a.s * sT[l16][jj + 2 * q] : 0.f;
        const float hi = (jj + 2 * q + 1 < a.r) ? a.s * sT[l16][jj + 2 * q + 1] : 0.f;
        tv[q] = pack_bf16x2(lo, hi);
      }
      const bf16x8_t ta = as_bf16x8(tv);
#pragma unroll
      for (int t = 0; t < kTiles; ++t) {
        const int rl = wave * 16 * kTiles + 16 * t + l16;
        uint4 bw;
        if (b_staged) {
          bw = (jj < a.r) ? sB[rl][jj / 8] : make_uint4(0, 0, 0, 0);
        } else {
          const int64_t n = row0 + rl;
          uint32_t e[8];
#pragma unroll
          for (int q = 0; q < 8; ++q)
            e[q] = __builtin_amdgcn_raw_buffer_load_b16(rb, (jj + q < a.r) ? (int)((n * a.r + jj + q) * 2) : (int)kOOB, 0, 0);
          bw = make_uint4((e[0] & 0xFFFFu) | (e[1] << 16), (e[2] & 0xFFFFu) | (e[3] << 16),
                          (e[4] & 0xFFFFu) | (e[5] << 16), (e[6] & 0xFFFFu) | (e[7] << 16));
        }
        acc[t] = mfma16x16x32(ta, as_bf16x8(bw), acc[t]);
      }
    }

  }  // general path

  // ---- output: D[m][n] -- lane holds rows m = 4g + v of column n
  if (a.ksplit == 1) {
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
      const int64_t n = row0 + wave * 16 * kTiles + 16 * t + l16;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t m = 4 * g + v;
        if (m < M && n < N) a.Y[m * N + n] = (uint16_t)(pack_bf16x2(acc[t][v], 0.f) & 0xFFFFu);
      }
    }
    if (a.T_save && grp == 0) {
      for (int i = tid; i < M * a.r; i += kThreads)
        a.T_save[i] = (uint16_t)(pack_bf16x2(sT[i / a.r][i % a.r], 0.f) & 0xFFFFu);
    }
    return;
  }
#pragma unroll
  for (int t = 0; t < kTiles; ++t) {
    const int64_t n = row0 + wave * 16 * kTiles + 16 * t + l16;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t m = 4 * g + v;
      if (m < M && n < N) publish(a.part + ((int64_t)ks * M + m) * N + n, acc[t][v]);
    }
  }
  if (grp == 0) {
    for (int i = tid; i < M * a.r; i += kThreads) publish(a.tpart + (int64_t)ks * M * a.r + i, sT[i / a.r][i % a.r]);
  }
  // every partial store of this workgroup has completed before its counter increment
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    const unsigned int old = __hip_atomic_fetch_add(&a.counters[grp], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = (old + 1u == (unsigned int)a.ksplit) ? 1u : 0u;
    if (s_last) __hip_atomic_store(&a.counters[grp], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!s_last) return;
  // last workgroup of this row group: fixed-order sum of the partials.  With one output per
  // thread, kSumU partials per round trip; with more, the loads of up to kSumOut outputs per
  // thread in flight together.
  const int64_t nrows = (row0 + kRows <= N) ? kRows : N - row0;
  if (M * nrows <= kThreads) {
    if (tid < M * nrows) {
      int m, nn;
      split_out(tid, (int)nrows, m, nn);
      const int64_t n = row0 + nn;
      a.Y[m * N + n] = (uint16_t)(pack_bf16x2(sum_published(a.part + m * N + n, a.ksplit, M * N), 0.f) & 0xFFFFu);
    }
  } else {
    for (int64_t i0 = tid; i0 < M * nrows; i0 += (int64_t)kThreads * kSumOut) {
      float sum[kSumOut];
      sum_published_n(a.part, i0, M * nrows, nrows, row0, N, a.ksplit, M * N, sum);
#pragma unroll
      for (int o = 0; o < kSumOut; ++o) {
        const int64_t i = i0 + (int64_t)o * kThreads;
        int m, nn;
        split_out((int)i, (int)nrows, m, nn);
        if (i < M * nrows) a.Y[(int64_t)m * N + row0 + nn] = (uint16_t)(pack_bf16x2(sum[o], 0.f) & 0xFFFFu);
      }
    }
  }
  if (a.T_save && grp == 0) {
    for (int i = tid; i < M * a.r; i += kThreads)
      a.T_save[i] = (uint16_t)(pack_bf16x2(sum_published(a.tpart + i, a.ksplit, M * a.r), 0.f) & 0xFFFFu);
  }
}

}  // namespace

int32_t gemv_ksplit(int64_t N, int64_t K) {
  const int64_t groups = (N + kRows - 1) / kRows;
  const int64_t nb_row = K / kBlock1;
  const int64_t want = (256 + groups - 1) / groups;
  int32_t ks = 1;
  while (ks < want && ks * 2 <= nb_row && ks < kMaxSplit) ks *= 2;
  return ks;
}

int64_t gemv_groups(int64_t N) { return (N + kRows - 1) / kRows; }

hipError_t launch_gemv_fwd(const uint32_t* codes, const uint8_t* code8, const float* c2s,
                           const float* mu, int64_t N, int64_t K, const uint16_t* X, int64_t M,
                           const uint16_t* A, const uint16_t* B, int32_t r, float s, uint16_t* Y,
                           uint16_t* T_save, float* part, float* tpart, unsigned int* counters,
                           const Nf4Tables& T, hipStream_t st) {
  GemvArgs a;
  a.codes = reinterpret_cast<const uint8_t*>(codes);
  a.code8 = code8;
  a.c2s = c2s;
  a.mu = mu;
  a.N = N;
  a.K = K;
  a.X = X;
  a.M = M;
  a.A = A;
  a.B = B;
  a.r = r;
  a.s = s;
  a.Y = Y;
  a.T_save = T_save;
  a.part = part;
  a.tpart = tpart;
  a.counters = counters;
  a.ksplit = gemv_ksplit(N, K);
  const int64_t nb_row = K / kBlock1;
  a.nbs = (int32_t)((nb_row + a.ksplit - 1) / a.ksplit);
  dim3 grid((unsigned)gemv_groups(N), (unsigned)a.ksplit);
  LaunchTimer t(3, st);
  // A full single chunk per workgroup: adapter part first, under the code transfer.  With
  // fewer blocks the codes land almost at once and the reordering only adds latency, so those
  // keep the chunk loop.
  const bool one = a.nbs == kChunk;
  if (r <= 16 && one) hipExtLaunchKernelGGL((k_gemv_fused<1, true>), grid, dim3(kThreads), 0, st, t.start, t.stop, 0, a, T);
  else if (r <= 16) hipExtLaunchKernelGGL((k_gemv_fused<1, false>), grid, dim3(kThreads), 0, st, t.start, t.stop, 0, a, T);
  else if (r <= 32 && one) hipExtLaunchKernelGGL((k_gemv_fused<2, true>), grid, dim3(kThreads), 0, st, t.start, t.stop, 0, a, T);
  else if (r <= 32) hipExtLaunchKernelGGL((k_gemv_fused<2, false>), grid, dim3(kThreads), 0, st, t.start, t.stop, 0, a, T);
  else if (r <= 64) hipExtLaunchKernelGGL((k_gemv_fused<4, false>), grid, dim3(kThreads), 0, st, t.start, t.stop, 0, a, T);
  else hipExtLaunchKernelGGL((k_gemv_fused<8, false>), grid, dim3(kThreads), 0, st, t.start, t.stop, 0, a, T);
  return hipGetLastError();
}

}  // namespace qlora
