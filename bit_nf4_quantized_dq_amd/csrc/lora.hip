// LoRA side-path kernels.  "QLoRA -- Fine-Tuning a 65B Model on One GPU", "Prerequisite:
// LoRA": A [r, d_in] projects the input down to r dimensions, B [d_out, r] expands it;
// "Where the gradients actually go": only A and B receive gradients.  "QLoRA: Quantize
// Base Weights to 4-Bit", Section 3: the branch is scaled by alpha/r.
//
// down : out[m][j] = sum_k P[m][k] Q(j, k)                    (T = X A^T, G = dY B)
//        Q is [R, Kd] (A) or [Kd, R] (B).  One workgroup owns 16*MT tokens and all R
//        outputs over the whole reduction (no partials); 8 wavefronts take interleaved
//        32-wide slabs and their sums meet in LDS in a fixed order.
// grad : out(j, c) = scale * sum_m U[m][j] V[m][c]            (dA = s G^T X, dB = s dY^T T)
//        One workgroup owns 64 columns c and a slice of the tokens; the slices' FP32 sums
//        are combined in a fixed order by the last workgroup of the column tile to finish
//        (arrival counters in the caller's workspace, one per column tile, reset to zero by
//        that workgroup; products with their own counters may run concurrently).
//
// Both use MFMA 16x16x32 BF16.  Operands whose reduction index is strided in memory (Q as
// [Kd, R], U and V) are staged in LDS row-major and read with ds_read_b64_tr_b16: within
// each 16-lane group, lane i receives element (i % 4) of the 8 bytes addressed by lanes
// i/4, i/4 + 4, i/4 + 8, i/4 + 12.  If lane j addresses row k0 + j/4, columns 4 (j % 4) .. +3
// of a tile with 16 columns, lane i therefore receives rows k0 .. k0+3 of column i, and two
// such reads give the 8 consecutive reduction indices of an MFMA operand.
#include "decode_tiles.h"
#include "qlora_host.h"

namespace qlora {

namespace {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

constexpr int kSumU = 16;                 // partials loaded together before they are added

// 8 consecutive rows k0 + 8 (lane >> 4) .. +7 of column (lane & 15) of an LDS tile with 16
// columns and a row pitch of `pitch` bytes (rows k0 .. k0 + 31).
__device__ __forceinline__ bf16x8_t tr_operand(const char* tile, int pitch, int lane) {
  const int j = lane & 15, g = lane >> 4;
  const char* p0 = tile + (8 * g + (j >> 2)) * pitch + 8 * (j & 3);
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p0));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p0 + 4 * pitch));
  bf16x8_t r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}

__device__ __forceinline__ uint16_t to_bf16(float v) { return (uint16_t)(pack_bf16x2(v, 0.f) & 0xFFFFu); }

// ---------------------------------------------------------------- down-projection
constexpr int kDownThreads = 512;
constexpr int kDownWaves = kDownThreads / 64;

// LDS of one down-projection workgroup: per wavefront, the QT staging of one slab (JT tiles
// of 32 rows x 16 columns); reused for the cross-wavefront sums.
template <int JT, int MT>
constexpr int down_lds_bytes() {
  return kDownWaves * JT * MT * 64 * 16 > kDownWaves * JT * 1024 ? kDownWaves * JT * MT * 64 * 16
                                                                   : kDownWaves * JT * 1024;
}

// Workgroup wg of the down-projection: tokens 16 MT wg .. +16 MT.  JT = ceil(R / 16) tiles of
// outputs, all held by every wavefront.
template <int JT, int MT, bool QT, int D>
__device__ __forceinline__ void down_body(const uint16_t* __restrict__ P, const uint16_t* __restrict__ Q, int64_t M,
                                          int32_t R, int64_t Kd, float scale, uint16_t* __restrict__ out_s,
                                          uint16_t* __restrict__ out_u, int64_t wg, char* smem) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t m0 = wg * 16 * MT;
  const int kk = 8 * (lane >> 4);
  const rsrc_t rp = make_rsrc(P + m0 * Kd, (M - m0) * Kd * 2);
  const rsrc_t rq = make_rsrc(Q, (int64_t)R * Kd * 2);
  f32x4_t acc[JT][MT];
#pragma unroll
  for (int t = 0; t < JT; ++t)
#pragma unroll
    for (int u = 0; u < MT; ++u) acc[t][u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  char* qs = smem + wave * JT * 1024;  // QT: this wavefront's slab, JT tiles of [32][16] BF16
  const int64_t nslab = (Kd + 31) / 32;
  // D slabs per pass (chosen at launch from the slabs per wavefront): all their global loads
  // are issued before the first is used, and no register buffer is carried across passes
  for (int64_t s0 = wave; s0 < nslab; s0 += (int64_t)kDownWaves * D) {
    uint4 pv[D][MT];
    uint4 qv[D][JT];
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int64_t s = s0 + (int64_t)kDownWaves * d;
      const int64_t k = 32 * s + kk;
      const bool kok = s < nslab && k < Kd;
#pragma unroll
      for (int u = 0; u < MT; ++u) {
        const int64_t row = 16 * u + (lane & 15);
        pv[d][u] = bload16(rp, (kok && m0 + row < M) ? (uint32_t)((row * Kd + k) * 2) : kOOB);
      }
      if (!QT) {
#pragma unroll
        for (int t = 0; t < JT; ++t) {
          const int j = 16 * t + (lane & 15);
          qv[d][t] = bload16(rq, (kok && j < R) ? (uint32_t)(((int64_t)j * Kd + k) * 2) : kOOB);
        }
      } else {
        // rows k = 32 s + (lane >> 1), columns 8 (lane & 1) .. +7 of every tile
        const int64_t kr = 32 * s + (lane >> 1);
        const bool rok = s < nslab && kr < Kd;
#pragma unroll
        for (int t = 0; t < JT; ++t) {
          const int j = 16 * t + 8 * (lane & 1);
          if ((R & 7) == 0) {  // 16-byte row pieces
            qv[d][t] = bload16(rq, (rok && j < R) ? (uint32_t)((kr * R + j) * 2) : kOOB);
          } else {
            uint32_t e[8];
#pragma unroll
            for (int q = 0; q < 8; ++q)
              e[q] = __builtin_amdgcn_raw_buffer_load_b16(rq, (rok && j + q < R) ? (int)((kr * R + j + q) * 2) : (int)kOOB, 0, 0);
            qv[d][t] = make_uint4((e[0] & 0xFFFFu) | (e[1] << 16), (e[2] & 0xFFFFu) | (e[3] << 16),
                                  (e[4] & 0xFFFFu) | (e[5] << 16), (e[6] & 0xFFFFu) | (e[7] << 16));
          }
        }
      }
    }
    // Every slab of the pass is used, also those past the end (their loads read as zero), so
    // no load sits behind a branch that the compiler could sink it into.
#pragma unroll
    for (int d = 0; d < D; ++d) {
      bf16x8_t qa[JT];
      if (!QT) {
#pragma unroll
        for (int t = 0; t < JT; ++t) qa[t] = as_bf16x8(qv[d][t]);
      } else {
        // the wavefront's LDS tiles are reused slab after slab; its LDS accesses run in order
        asm volatile("" ::: "memory");
#pragma unroll
        for (int t = 0; t < JT; ++t) *reinterpret_cast<uint4*>(qs + t * 1024 + (lane >> 1) * 32 + 16 * (lane & 1)) = qv[d][t];
        asm volatile("" ::: "memory");
#pragma unroll
        for (int t = 0; t < JT; ++t) qa[t] = tr_operand(qs + t * 1024, 32, lane);
        asm volatile("" ::: "memory");
      }
#pragma unroll
      for (int t = 0; t < JT; ++t)
#pragma unroll
        for (int u = 0; u < MT; ++u) acc[t][u] = mfma16x16x32(qa[t], as_bf16x8(pv[d][u]), acc[t][u]);
    }
  }
  // fixed-order sum over the wavefronts
  __syncthreads();
  f32x4_t* red = reinterpret_cast<f32x4_t*>(smem);
#pragma unroll
  for (int t = 0; t < JT; ++t)
#pragma unroll
    for (int u = 0; u < MT; ++u) red[((wave * JT + t) * MT + u) * 64 + lane] = acc[t][u];
  __syncthreads();
  for (int i = threadIdx.x; i < JT * MT * 64; i += kDownThreads) {
    const int l = i & 63, u = (i >> 6) % MT, t = (i >> 6) / MT;
    f32x4_t sum = red[(t * MT + u) * 64 + l];
    for (int w = 1; w < kDownWaves; ++w) {
      const f32x4_t v = red[((w * JT + t) * MT + u) * 64 + l];
      sum[0] += v[0]; sum[1] += v[1]; sum[2] += v[2]; sum[3] += v[3];
    }
    // D[j][m]: lane l holds rows j = 4 (l >> 4) + v of column m = l & 15
    const int64_t m = m0 + 16 * u + (l & 15);
    if (m >= M) continue;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int j = 16 * t + 4 * (l >> 4) + v;
      if (j >= R) continue;
      if (out_s) out_s[m * R + j] = to_bf16(sum[v] * scale);
      if (out_u) out_u[m * R + j] = to_bf16(sum[v]);
    }
  }
}

// grid: ceil(M / (16 MT))
template <int JT, int MT, bool QT, int D>
__global__ __launch_bounds__(kDownThreads) void k_lora_down(const uint16_t* __restrict__ P,
                                                            const uint16_t* __restrict__ Q, int64_t M,
                                                            int32_t R, int64_t Kd, float scale,
                                                            uint16_t* __restrict__ out_s,
                                                            uint16_t* __restrict__ out_u) {
  __shared__ __attribute__((aligned(16))) char smem[down_lds_bytes<JT, MT>()];
  down_body<JT, MT, QT, D>(P, Q, M, R, Kd, scale, out_s, out_u, blockIdx.x, smem);
}

// The step's two prologues pair a down-projection with a decode of the weight: the two are
// independent and each bound by HBM, so one launch runs both.  The first n_down workgroups
// project; the rest decode.
struct DownArgs {
  const uint16_t* P;
  const uint16_t* Q;
  int64_t M;
  int32_t R;
  int64_t Kd;
  float scale;
  uint16_t* out_s;
  uint16_t* out_u;
};
struct DecodeArgs {
  const uint32_t* codes;
  const uint8_t* code8;
  const float* c2s;
  const float* mu;
  uint16_t* out;
  int64_t N, K;
};

// Forward: T = X A^T, and the decoded copy w_hat [N, K] (kDecWords x 256 code words per
// workgroup).
template <int JT, int MT, int D, int DQ>
__global__ __launch_bounds__(kDownThreads) void k_fwd_prologue(DownArgs d, DecodeArgs e, int64_t n_down, Nf4Tables T) {
  __shared__ __attribute__((aligned(16))) char smem[down_lds_bytes<JT, MT>()];
  if ((int64_t)blockIdx.x < n_down) {
    down_body<JT, MT, false, D>(d.P, d.Q, d.M, d.R, d.Kd, d.scale, d.out_s, d.out_u, blockIdx.x, smem);
    return;
  }
  decode_words<DQ, kDownThreads>(e.codes, e.code8, e.c2s, e.mu, reinterpret_cast<uint4*>(e.out), (int64_t)blockIdx.x - n_down,
                   threadIdx.x, e.N * e.K / 8, T);
}

// Backward: G = dY B, and the transposed decoded copy w_hat^T [K, N] (128 rows x 8 blocks per
// workgroup, decode_pairs_t; no LDS, so the decode takes none from the G role's workgroups).
template <int JT, int MT, int D, int DQ>
__global__ __launch_bounds__(kDownThreads) void k_bwd_prologue(DownArgs d, DecodeArgs e, int64_t n_down, Nf4Tables T) {
  __shared__ __attribute__((aligned(16))) char smem[down_lds_bytes<JT, MT>()];
  if ((int64_t)blockIdx.x < n_down) {
    down_body<JT, MT, true, D>(d.P, d.Q, d.M, d.R, d.Kd, d.scale, d.out_s, d.out_u, blockIdx.x, smem);
    return;
  }
  // 32-bit group arithmetic (fewer than 2^31 groups): a 64-bit division here delayed the
  // decode's first loads
  constexpr int kBlocks = kDownThreads / 64;  // k blocks per workgroup
  const uint32_t groups_k = (uint32_t)((e.K / 64 + kBlocks - 1) / kBlocks);
  const uint32_t grp = (uint32_t)((int64_t)blockIdx.x - n_down);
  const uint32_t gn = grp / groups_k;
  decode_pairs_t<DQ, kDownThreads>(e.codes, e.code8, e.c2s, e.mu, e.out, e.N, e.K, T, (int64_t)gn,
                                   (int64_t)(grp - gn * groups_k), threadIdx.x);
}

// ---------------------------------------------------------------- gradients of A and B
constexpr int kGradThreads = 256;
constexpr int kGradWaves = kGradThreads / 64;
constexpr int kGradCols = 64;      // columns per workgroup (4 tiles of 16)
constexpr int kVTile = 32 * 32 + 64;  // bytes per staged [32][16] BF16 tile, padded (bank offset)

// One gradient product out = scale * U^T V (or its transpose): U [M, R], V [M, C].
struct GradArgs {
  const uint16_t* U;
  const uint16_t* V;
  int64_t M;
  int32_t R;
  int64_t C;
  int64_t mps;          // tokens per slice (a multiple of 32)
  float scale;
  int transposed;       // out is [C, R] instead of [R, C]
  float* part;          // [msplit][R][C] FP32 (msplit > 1)
  unsigned int* counters;
  uint16_t* out;
  int32_t msplit;
};

// The workgroup of column tile c_tile (64 columns) and token slice m_slice.  JT = ceil(R / 16).
template <int JT, int D>
__device__ __forceinline__ void grad_body(const GradArgs& g, int64_t c_tile, int64_t m_slice) {
  const uint16_t* __restrict__ U = g.U;
  const uint16_t* __restrict__ V = g.V;
  const int64_t M = g.M, C = g.C, mps = g.mps;
  const int32_t R = g.R;
  const float scale = g.scale;
  const int transposed = g.transposed;
  float* __restrict__ part = g.part;
  unsigned int* __restrict__ counters = g.counters;
  uint16_t* __restrict__ out = g.out;
  // per wavefront: 4 V tiles + JT U tiles of [32][16] BF16; reused for the cross-wave sums
  constexpr int kWaveBytes = (4 + JT) * kVTile;
  constexpr int kRedBytes = kGradWaves * JT * 4 * 64 * 16;
  __shared__ __attribute__((aligned(16))) char smem[kGradWaves * kWaveBytes > kRedBytes ? kGradWaves * kWaveBytes : kRedBytes];
  __shared__ bool s_last;
  // the wavefront index is uniform: keep it in a scalar register so the per-chunk buffer
  // descriptors below stay scalar
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t c0 = c_tile * kGradCols;
  const int64_t mbeg = m_slice * mps;
  const int64_t mend = (mbeg + mps < M) ? mbeg + mps : M;
  char* vt = smem + wave * kWaveBytes;  // 4 V tiles, then JT U tiles
  char* ut = vt + 4 * kVTile;
  f32x4_t acc[JT][4];
#pragma unroll
  for (int t = 0; t < JT; ++t)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[t][q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // wavefront w takes chunks of 32 tokens mbeg + 32 (w + 4 i), D chunks per pass (chosen at
  // launch from the chunks per wavefront): all their global loads are issued before the
  // first chunk is staged, so D chunks stay in flight
  const bool uvec = (R & 7) == 0;
  for (int64_t mc0 = mbeg + 32 * wave; mc0 < mend; mc0 += (int64_t)32 * kGradWaves * D) {
    uint4 vv[D][4];     // V chunk [32][64]: lane -> row 8 i + (lane >> 3), columns 8 (lane & 7) .. +7
    uint4 uw[D][JT];    // U chunk [32][16 JT]: lane -> row lane >> 1, columns 16 t + 8 (lane & 1) .. +7
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int64_t mc = mc0 + (int64_t)32 * kGradWaves * d;
      // descriptors based at the chunk's first token: in-chunk offsets stay below 32 rows,
      // whatever M * C is (rows at or past mend read as zero)
      const int64_t live = mend - mc;
      const rsrc_t rv = make_rsrc(V + mc * C, live * C * 2);
      const rsrc_t ru = make_rsrc(U + mc * R, live * (int64_t)R * 2);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t ml = 8 * i + (lane >> 3);
        const int64_t c = c0 + 8 * (lane & 7);
        vv[d][i] = bload16(rv, (ml < live && c < C) ? (uint32_t)((ml * C + c) * 2) : kOOB);
      }
      const int64_t ml = lane >> 1;
#pragma unroll
      for (int t = 0; t < JT; ++t) {
        const int j = 16 * t + 8 * (lane & 1);
        if (uvec) {
          uw[d][t] = bload16(ru, (ml < live && j < R) ? (uint32_t)((ml * R + j) * 2) : kOOB);
        } else {
          uint32_t e[8];
#pragma unroll
          for (int q = 0; q < 8; ++q)
            e[q] = __builtin_amdgcn_raw_buffer_load_b16(ru, (ml < live && j + q < R) ? (int)((ml * R + j + q) * 2) : (int)kOOB, 0, 0);
          uw[d][t] = make_uint4((e[0] & 0xFFFFu) | (e[1] << 16), (e[2] & 0xFFFFu) | (e[3] << 16),
                                (e[4] & 0xFFFFu) | (e[5] << 16), (e[6] & 0xFFFFu) | (e[7] << 16));
        }
      }
    }
    // Every chunk of the pass is used, also those past the end (their loads read as zero),
    // so no load sits behind a branch that the compiler could sink it into.
#pragma unroll
    for (int d = 0; d < D; ++d) {
      // the wavefront's LDS tiles are reused chunk after chunk; its LDS accesses run in order
      asm volatile("" ::: "memory");
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 8 * i + (lane >> 3), ct = (lane & 7) >> 1, half = lane & 1;
        *reinterpret_cast<uint4*>(vt + ct * kVTile + row * 32 + 16 * half) = vv[d][i];
      }
#pragma unroll
      for (int t = 0; t < JT; ++t) *reinterpret_cast<uint4*>(ut + t * kVTile + (lane >> 1) * 32 + 16 * (lane & 1)) = uw[d][t];
      asm volatile("" ::: "memory");
      bf16x8_t a[JT], b[4];
#pragma unroll
      for (int t = 0; t < JT; ++t) a[t] = tr_operand(ut + t * kVTile, 32, lane);
#pragma unroll
      for (int q = 0; q < 4; ++q) b[q] = tr_operand(vt + q * kVTile, 32, lane);
      asm volatile("" ::: "memory");
#pragma unroll
      for (int t = 0; t < JT; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[t][q] = mfma16x16x32(a[t], b[q], acc[t][q]);
    }
  }
  // fixed-order sum over the wavefronts: D[j][c], lane l holds j = 4 (l >> 4) + v, c = l & 15
  __syncthreads();
  f32x4_t* red = reinterpret_cast<f32x4_t*>(smem);
#pragma unroll
  for (int t = 0; t < JT; ++t)
#pragma unroll
    for (int q = 0; q < 4; ++q) red[((wave * JT + t) * 4 + q) * 64 + lane] = acc[t][q];
  __syncthreads();
  const int32_t msplit = g.msplit;
  // one (t, q, lane) item per thread pass: JT * 4 * 64 items
  for (int i = threadIdx.x; i < JT * 4 * 64; i += kGradThreads) {
    const int l = i & 63, q = (i >> 6) & 3, t = i >> 8;
    f32x4_t sum = red[(t * 4 + q) * 64 + l];
    for (int w = 1; w < kGradWaves; ++w) {
      const f32x4_t v = red[((w * JT + t) * 4 + q) * 64 + l];
      sum[0] += v[0]; sum[1] += v[1]; sum[2] += v[2]; sum[3] += v[3];
    }
    const int64_t c = c0 + 16 * q + (l & 15);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int j = 16 * t + 4 * (l >> 4) + v;
      if (j >= R || c >= C) continue;
      if (msplit == 1) {
        const uint16_t b16 = to_bf16(sum[v] * scale);
        if (transposed) out[c * R + j] = b16;
        else out[(int64_t)j * C + c] = b16;
      } else {
        __hip_atomic_store(part + (m_slice * R + j) * C + c, sum[v], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_SYSTEM);
      }
    }
  }
  if (msplit == 1) return;
  // every partial store of this workgroup has completed before its counter increment
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned int old = __hip_atomic_fetch_add(&counters[c_tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = old + 1u == (unsigned int)msplit;
    if (s_last) __hip_atomic_store(&counters[c_tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!s_last) return;
  // last workgroup of this column tile: fixed-order sum of the slices
  const int64_t ncol = (c0 + kGradCols <= C) ? kGradCols : C - c0;
  for (int64_t i = threadIdx.x; i < (int64_t)R * ncol; i += kGradThreads) {
    // 32-bit (R ncol <= 128 kGradCols), a shift for a whole tile: a 64-bit division is a long
    // sequence, and this runs in the launch's tail
    const int ii = (int)i, nc = (int)ncol;
    const int32_t j = nc == kGradCols ? (int32_t)((unsigned)ii / (unsigned)kGradCols) : (int32_t)((unsigned)ii / (unsigned)nc);
    const int64_t c = c0 + (ii - j * nc);
    const float* p = part + (int64_t)j * C + c;
    float s = 0.f;
    for (int32_t k0 = 0; k0 < msplit; k0 += kSumU) {
      float v[kSumU];
#pragma unroll
      for (int u = 0; u < kSumU; ++u)
        v[u] = (k0 + u < msplit) ? __hip_atomic_load(p + (int64_t)(k0 + u) * R * C, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM)
                                 : 0.f;
#pragma unroll
      for (int u = 0; u < kSumU; ++u) s += v[u];
    }
    const uint16_t b16 = to_bf16(s * scale);
    if (transposed) out[c * R + j] = b16;
    else out[(int64_t)j * C + c] = b16;
  }
}

// grid (ceil(C / 64), msplit)
template <int JT, int D>
__global__ __launch_bounds__(kGradThreads) void k_lora_grad(GradArgs g) {
  grad_body<JT, D>(g, blockIdx.x, blockIdx.y);
}

// Two independent products in one launch (dA and dB of one backward), blockIdx.z selecting:
// grid (max column tiles, max slices, 2); workgroups past a product's own grid return.
template <int JT, int D>
__global__ __launch_bounds__(kGradThreads) void k_lora_grad2(GradArgs g0, GradArgs g1) {
  const GradArgs& g = blockIdx.z ? g1 : g0;
  if ((int64_t)blockIdx.x * kGradCols >= g.C || (int32_t)blockIdx.y >= g.msplit) return;
  grad_body<JT, D>(g, blockIdx.x, blockIdx.y);
}

// Batch depth: slabs (or token chunks) per pass, at most the wavefront's share and at most
// kMaxD (the register budget of the loads held at once).
inline int batch_depth(int64_t per_wave, int max_d) {
  int d = 1;
  while (d < max_d && d < per_wave) d *= 2;
  return d;
}

template <int JT, int MT, bool QT>
hipError_t down_launch(const uint16_t* P, const uint16_t* Q, int64_t M, int32_t R, int64_t Kd, float scale,
                       uint16_t* out_s, uint16_t* out_u, hipStream_t s) {
  const int64_t grid = (M + 16 * MT - 1) / (16 * MT);
  constexpr int kMaxD = (JT + MT <= 2) ? 16 : (JT + MT <= 3 ? 8 : (JT + MT <= 6 ? 4 : 2));  // <= 128 VGPRs
  const int d = batch_depth(((Kd + 31) / 32 + kDownWaves - 1) / kDownWaves, kMaxD);
  LaunchTimer t(6, s);
  auto go = [&](auto kern) {
    hipExtLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kDownThreads), 0, s, t.start, t.stop, 0, P, Q, M, R, Kd, scale,
                          out_s, out_u);
  };
  if (d >= 16 && kMaxD >= 16) go(k_lora_down<JT, MT, QT, (kMaxD >= 16 ? 16 : 1)>);
  else if (d >= 8 && kMaxD >= 8) go(k_lora_down<JT, MT, QT, (kMaxD >= 8 ? 8 : 1)>);
  else if (d >= 4 && kMaxD >= 4) go(k_lora_down<JT, MT, QT, (kMaxD >= 4 ? 4 : 1)>);
  else if (d >= 2) go(k_lora_down<JT, MT, QT, 2>);
  else go(k_lora_down<JT, MT, QT, 1>);
  return hipGetLastError();
}

// Gradient product arguments: msplit token slices of mps tokens; one arrival counter per
// column tile at `counters`.
GradArgs grad_args(const uint16_t* U, const uint16_t* V, int64_t M, int32_t R, int64_t C, float scale, int transposed,
                   float* part, unsigned int* counters, uint16_t* out) {
  GradArgs g;
  g.U = U;
  g.V = V;
  g.M = M;
  g.R = R;
  g.C = C;
  g.msplit = lora_grad_msplit(M, C);
  g.mps = ((M + g.msplit - 1) / g.msplit + 31) / 32 * 32;
  g.scale = scale;
  g.transposed = transposed;
  g.part = part;
  g.counters = counters;
  g.out = out;
  return g;
}

// Loads of D token chunks are held at once: D is chosen from the chunks per wavefront.
// The paired prologue launches (E4M3 constants).  Depth of the down-projection's loads as in
// down_launch, at most 8 for the transposed operand (registers shared with the decode role).
template <int JT, int MT, bool BWD>
hipError_t prologue_launch(const DownArgs& dn, const DecodeArgs& de, const Nf4Tables& T, hipStream_t s) {
  const int64_t n_down = (dn.M + 16 * MT - 1) / (16 * MT);
  const int64_t n_dec = BWD ? ((de.K / 64 + kDownThreads / 64 - 1) / (kDownThreads / 64)) * ((de.N + kTRows - 1) / kTRows)
                            : (de.N * de.K / 8 + kDownThreads * kDecWords - 1) / (kDownThreads * kDecWords);
  constexpr int kMaxD = BWD ? ((JT + MT <= 3) ? 8 : (JT + MT <= 6 ? 4 : 2))
                            : ((JT + MT <= 2) ? 16 : (JT + MT <= 3 ? 8 : (JT + MT <= 6 ? 4 : 2)));
  const int d = batch_depth(((dn.Kd + 31) / 32 + kDownWaves - 1) / kDownWaves, kMaxD);
  LaunchTimer t(BWD ? 8 : 2, s);
  auto go = [&](auto kern) {
    hipExtLaunchKernelGGL(kern, dim3((unsigned)(n_down + n_dec)), dim3(kDownThreads), 0, s, t.start, t.stop, 0, dn, de,
                          n_down, T);
  };
  if (BWD) {
    if (d >= 8 && kMaxD >= 8) go(k_bwd_prologue<JT, MT, (kMaxD >= 8 ? 8 : 1), kDqE4M3>);
    else if (d >= 4 && kMaxD >= 4) go(k_bwd_prologue<JT, MT, (kMaxD >= 4 ? 4 : 1), kDqE4M3>);
    else go(k_bwd_prologue<JT, MT, 2, kDqE4M3>);
  } else {
    if (d >= 16 && kMaxD >= 16) go(k_fwd_prologue<JT, MT, (kMaxD >= 16 ? 16 : 1), kDqE4M3>);
    else if (d >= 8 && kMaxD >= 8) go(k_fwd_prologue<JT, MT, (kMaxD >= 8 ? 8 : 1), kDqE4M3>);
    else if (d >= 4 && kMaxD >= 4) go(k_fwd_prologue<JT, MT, (kMaxD >= 4 ? 4 : 1), kDqE4M3>);
    else go(k_fwd_prologue<JT, MT, 2, kDqE4M3>);
  }
  return hipGetLastError();
}

template <bool BWD>
hipError_t prologue_dispatch(const DownArgs& dn, const DecodeArgs& de, const Nf4Tables& T, hipStream_t s) {
  if (dn.R <= 16) return prologue_launch<1, 1, BWD>(dn, de, T, s);
  if (dn.R <= 32) return prologue_launch<2, 1, BWD>(dn, de, T, s);
  if (dn.R <= 64) return prologue_launch<4, 2, BWD>(dn, de, T, s);
  return prologue_launch<8, 2, BWD>(dn, de, T, s);
}

template <int JT>
int grad_depth(int64_t mps) {
  constexpr int kMaxD = JT <= 2 ? 8 : (JT <= 4 ? 4 : 2);  // <= 192 VGPRs of loads
  return batch_depth((mps / 32 + kGradWaves - 1) / kGradWaves, kMaxD);
}

template <int JT>
hipError_t grad_launch(const GradArgs& g0, const GradArgs* g1, hipStream_t s) {
  constexpr int kMaxD = JT <= 2 ? 8 : (JT <= 4 ? 4 : 2);
  int d = grad_depth<JT>(g0.mps);
  int64_t tiles = (g0.C + kGradCols - 1) / kGradCols;
  int32_t ms = g0.msplit;
  if (g1) {
    const int d1 = grad_depth<JT>(g1->mps);
    d = d1 < d ? d1 : d;
    const int64_t t1 = (g1->C + kGradCols - 1) / kGradCols;
    tiles = t1 > tiles ? t1 : tiles;
    ms = g1->msplit > ms ? g1->msplit : ms;
  }
  LaunchTimer t(7, s);
  auto go = [&](auto k1, auto k2) {
    if (g1)
      hipExtLaunchKernelGGL(k2, dim3((unsigned)tiles, (unsigned)ms, 2), dim3(kGradThreads), 0, s, t.start, t.stop, 0, g0,
                            *g1);
    else
      hipExtLaunchKernelGGL(k1, dim3((unsigned)tiles, (unsigned)ms), dim3(kGradThreads), 0, s, t.start, t.stop, 0, g0);
  };
  if (d >= 8 && kMaxD >= 8) go(k_lora_grad<JT, (kMaxD >= 8 ? 8 : 1)>, k_lora_grad2<JT, (kMaxD >= 8 ? 8 : 1)>);
  else if (d >= 4 && kMaxD >= 4) go(k_lora_grad<JT, (kMaxD >= 4 ? 4 : 1)>, k_lora_grad2<JT, (kMaxD >= 4 ? 4 : 1)>);
  else if (d >= 2) go(k_lora_grad<JT, 2>, k_lora_grad2<JT, 2>);
  else go(k_lora_grad<JT, 1>, k_lora_grad2<JT, 1>);
  return hipGetLastError();
}

hipError_t grad_dispatch(const GradArgs& g0, const GradArgs* g1, hipStream_t s) {
  const int32_t R = g0.R;
  if (R <= 16) return grad_launch<1>(g0, g1, s);
  if (R <= 32) return grad_launch<2>(g0, g1, s);
  if (R <= 64) return grad_launch<4>(g0, g1, s);
  return grad_launch<8>(g0, g1, s);
}

}  // namespace

hipError_t launch_lora_down(const uint16_t* P, const uint16_t* Q, int q_transposed, int64_t M, int32_t R, int64_t Kd,
                            float scale, uint16_t* out_s, uint16_t* out_u, hipStream_t s) {
  // tokens per workgroup grow with R so that Q (re-read by every workgroup) stays amortized
  if (q_transposed) {
    if (R <= 16) return down_launch<1, 1, true>(P, Q, M, R, Kd, scale, out_s, out_u, s);
    if (R <= 32) return down_launch<2, 1, true>(P, Q, M, R, Kd, scale, out_s, out_u, s);
    if (R <= 64) return down_launch<4, 2, true>(P, Q, M, R, Kd, scale, out_s, out_u, s);
    return down_launch<8, 2, true>(P, Q, M, R, Kd, scale, out_s, out_u, s);
  }
  if (R <= 16) return down_launch<1, 1, false>(P, Q, M, R, Kd, scale, out_s, out_u, s);
  if (R <= 32) return down_launch<2, 1, false>(P, Q, M, R, Kd, scale, out_s, out_u, s);
  if (R <= 64) return down_launch<4, 2, false>(P, Q, M, R, Kd, scale, out_s, out_u, s);
  return down_launch<8, 2, false>(P, Q, M, R, Kd, scale, out_s, out_u, s);
}

hipError_t launch_fwd_prologue(const uint16_t* X, const uint16_t* A, int64_t M, int32_t R, int64_t K, float scale,
                               uint16_t* t_s, uint16_t* t_u, const uint32_t* codes, const uint8_t* code8,
                               const float* c2s, const float* mu, int64_t N, uint16_t* w_out, const Nf4Tables& T,
                               hipStream_t s) {
  const DownArgs dn{X, A, M, R, K, scale, t_s, t_u};
  const DecodeArgs de{codes, code8, c2s, mu, w_out, N, K};
  return prologue_dispatch<false>(dn, de, T, s);
}

hipError_t launch_bwd_prologue(const uint16_t* dY, const uint16_t* B, int64_t M, int32_t R, int64_t N, float scale,
                               uint16_t* g_s, uint16_t* g_u, const uint32_t* codes, const uint8_t* code8,
                               const float* c2s, const float* mu, int64_t K, uint16_t* wt_out, const Nf4Tables& T,
                               hipStream_t s) {
  const DownArgs dn{dY, B, M, R, N, scale, g_s, g_u};
  const DecodeArgs de{codes, code8, c2s, mu, wt_out, N, K};
  return prologue_dispatch<true>(dn, de, T, s);
}

int32_t lora_grad_msplit(int64_t M, int64_t C) {
  const int64_t tiles = (C + kGradCols - 1) / kGradCols;
  int32_t ms = 1;
  while (tiles * ms < 256 && (int64_t)ms * 2 * 128 <= M && ms < 64) ms *= 2;
  return ms;
}

hipError_t launch_lora_grad(const uint16_t* U, const uint16_t* V, int64_t M, int32_t R, int64_t C, float scale,
                            int transposed, float* part, unsigned int* counters, uint16_t* out, hipStream_t s) {
  const GradArgs g = grad_args(U, V, M, R, C, scale, transposed, part, counters, out);
  return grad_dispatch(g, nullptr, s);
}

hipError_t launch_lora_grad2(const uint16_t* U0, const uint16_t* V0, int64_t C0, int transposed0, float* part0,
                             unsigned int* counters0, uint16_t* out0, const uint16_t* U1, const uint16_t* V1,
                             int64_t C1, int transposed1, float* part1, unsigned int* counters1, uint16_t* out1,
                             int64_t M, int32_t R, float scale, hipStream_t s) {
  const GradArgs g0 = grad_args(U0, V0, M, R, C0, scale, transposed0, part0, counters0, out0);
  const GradArgs g1 = grad_args(U1, V1, M, R, C1, scale, transposed1, part1, counters1, out1);
  return grad_dispatch(g0, &g1, s);
}

}  // namespace qlora
