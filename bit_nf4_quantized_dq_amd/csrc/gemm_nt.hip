// BF16 MFMA GEMM over a dequantized weight copy, for many tokens.
//
// "QLoRA: Quantize Base Weights to 4-Bit", Section 3: the quantized weights are expanded to
// BF16 and multiplied in BF16.  For a large token count every weight would otherwise be
// decoded once per token tile, so the weight is decoded once into a BF16 scratch copy
// (w_hat for the forward, w_hat^T for dX -- the same bit-exact decode as everywhere else)
// and this kernel runs the plain product plus the adapter term:
//
//   C[f][m] = sum_k A[f][k] * B[m][k]  +  sum_j Wl[f][j] * L[m][j]       (FP32 accumulate)
//
//   forward : A = w_hat [N, K], B = X [M, K], Wl = B_lora [N, r], L = s T;   C = Y^T
//   dX      : A = w_hat^T [K, N], B = dY [M, N], Wl = A_lora^T, L = s G;     C = dX^T
// (C is stored token-major, i.e. as Y [M, N] / dX [M, K].)
//
// Tiling: 256 (f) x 256 (m) per workgroup, 8 wavefronts in a 2 x 4 grid of 128 x 64
// wavefront tiles (4 x 2 MFMA 32x32x16 tiles, 128 FP32 accumulators per lane), reduction
// step 32.  Both operand tiles stream through five-slot LDS rings (all 160 KB of LDS)
// filled by direct buffer->LDS loads issued three steps ahead, with one barrier per pair of
// steps (details at nt_step).  The step loop is unrolled ten times so that each ring slot
// is a distinct LDS array known at compile time, which lets the compiler wait only for the
// slot an access touches.  Rows are 4 chunks of
// 16 bytes, XOR-swizzled by (row >> 2) & 3: the LDS serves 16 lanes x 16 bytes per clock
// from 64 banks, and the 16 rows x one chunk of an MFMA operand read then cover all 256
// bytes exactly once; the ring writes (1 KB contiguous per load) are conflict-free anyway.  Out-of-range rows or
// reduction columns read as zero (raw buffer loads), so no tail needs a branch in the loop.
//
// Split reduction.  A product with few tiles (at most 128, e.g. a 1024-row projection at
// 2048 tokens: 32 tiles) would leave most CUs idle, so its reduction steps are dealt to
// ksplit workgroups per tile (blockIdx.z).  Each writes its FP32 partial tile to the
// workspace; k_sum_parts then adds the ksplit partials in a fixed order and rounds to BF16.
// The adapter slices run in split 0 only.
#include "qlora_device.h"
#include "qlora_host.h"

namespace qlora {
namespace {

constexpr int kThreads = 512;
constexpr int BF = 256;               // features (A rows) per tile
constexpr int BMT = 256;              // tokens (B rows) per tile
constexpr int BK = 32;                // reduction step
constexpr int kChunks = BK / 8;       // 16-byte chunks per LDS row
constexpr int kSlot = 256 * kChunks;  // 16-byte chunks per ring slot (16 KB)
constexpr int TI = 4, TJ = 2;         // 32x32 MFMA tiles per wavefront
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef f32x16_t Acc[TI][TJ];
typedef __attribute__((address_space(3))) void lds_void;

// Two rings of five 16 KB slots (160 KB, all of a CU's LDS).
constexpr int kRing = 5;
// A row offset past every tile (tiles are below 2^31 bytes and step offsets below 2^24), so
// a missing row reads zeros however the scalar step offset adds to it.
constexpr uint32_t kFarRow = 0xF0000000u;
__shared__ uint4 s_a0[kSlot], s_a1[kSlot], s_a2[kSlot], s_a3[kSlot], s_a4[kSlot];
__shared__ uint4 s_b0[kSlot], s_b1[kSlot], s_b2[kSlot], s_b3[kSlot], s_b4[kSlot];

template <int I> __device__ __forceinline__ uint4* abuf() {
  return I == 0 ? s_a0 : (I == 1 ? s_a1 : (I == 2 ? s_a2 : (I == 3 ? s_a3 : s_a4)));
}
template <int I> __device__ __forceinline__ uint4* bbuf() {
  return I == 0 ? s_b0 : (I == 1 ? s_b1 : (I == 2 ? s_b2 : (I == 3 ? s_b3 : s_b4)));
}

__device__ __forceinline__ f32x16_t mfma32(const bf16x8_t& a, const bf16x8_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kChunks + (chunk ^ ((row >> 2) & 3));
}

template <int N> __device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}
// Own LDS writes done, then the workgroup barrier (also a compiler memory barrier).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("s_barrier" ::: "memory");
}

// One operand ring: rows row0 .. row0+255 of a [rows_total, Kr] BF16 matrix.  Wavefront w
// fills rows 32w .. 32w+31 of a slot with 2 loads of 16 rows x 4 chunks; lane p of load j
// writes slot chunk (p & 3) of row 16(2w+j) + (p >> 2) and fetches the logical chunk the
// swizzle maps there.
struct Ring {
  rsrc_t r;
  uint32_t base[2];  // byte offset of the lane's chunk at reduction index 0; past the rows,
                     // kFarRow (whole steps) or kOOB
  uint32_t col[2];   // the lane's first reduction index within a step
  uint32_t Kr;
  uint32_t kbase;  // first reduction step of this workgroup's range
  uint32_t kmax;   // last reduction step of the whole product
  int wave;

  template <bool FULLK>
  __device__ __forceinline__ void init(const uint16_t* P, int64_t rows_total, int64_t row0, int64_t Kr_, int w,
                                       int lane, uint32_t kb0) {
    const int64_t rows = rows_total - row0 < 256 ? rows_total - row0 : 256;
    r = make_rsrc(P + row0 * Kr_, rows * Kr_ * 2);
    Kr = (uint32_t)Kr_;
    kbase = kb0;
    kmax = (uint32_t)((Kr_ + BK - 1) / BK) - 1u;
    wave = w;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int row = 16 * (2 * w + j) + (lane >> 2);
      const int lc = (lane & 3) ^ ((row >> 2) & 3);
      col[j] = 8 * lc;
      base[j] = row < rows ? (uint32_t)(row * Kr_ * 2 + 16 * lc) : (FULLK ? kFarRow : kOOB);
    }
  }
  template <bool FULLK>
  __device__ __forceinline__ void issue1(uint4* slot, uint32_t kb, int j) const {
    if (FULLK) {
      // whole steps only: the row offset stays in the lane's register and the step's column
      // offset goes in the scalar offset; steps past the product reload its last step
      const uint32_t kk = kbase + kb < kmax ? kbase + kb : kmax;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(slot + (2 * wave + j) * 64), 16, base[j], kk * (2 * BK), 0, 0);
    } else {
      const uint32_t k0 = (kbase + kb) * BK;
      const uint32_t off = (base[j] != kOOB && k0 + col[j] < Kr) ? base[j] + 2 * k0 : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(slot + (2 * wave + j) * 64), 16, off, 0, 0, 0);
    }
  }
  template <bool FULLK>
  __device__ __forceinline__ void issue(uint4* slot, uint32_t kb) const {
    issue1<FULLK>(slot, kb, 0);
    issue1<FULLK>(slot, kb, 1);
  }
};

// Operands of one 16-wide reduction step (ks = 0 or 1 of a 32-wide ring step).  Lane l
// supplies row (l & 31) of each operand tile and reduction indices 8*(l >> 5) .. +7.
struct Ops {
  bf16x8_t a[TI], b[TJ];
};
__device__ __forceinline__ void read_ops(const uint4* __restrict__ sa, const uint4* __restrict__ sb, int ks, int wf,
                                         int wmt, int l32, int h32, Ops& o) {
#pragma unroll
  for (int i = 0; i < TI; ++i) o.a[i] = as_bf16x8(sa[swz(wf + 32 * i + l32, 2 * ks + h32)]);
#pragma unroll
  for (int j = 0; j < TJ; ++j) o.b[j] = as_bf16x8(sb[swz(wmt + 32 * j + l32, 2 * ks + h32)]);
}
__device__ __forceinline__ void mma(const Ops& o, Acc& acc) {
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = mfma32(o.a[i], o.b[j], acc[i][j]);
}
// Half of mma(): tiles i = 2h, 2h + 1 (4 MFMAs).
__device__ __forceinline__ void mma_half(const Ops& o, int h, Acc& acc) {
#pragma unroll
  for (int i = 2 * h; i < 2 * h + 2; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = mfma32(o.a[i], o.b[j], acc[i][j]);
}
__device__ __forceinline__ void mma_step(const uint4* __restrict__ sa, const uint4* __restrict__ sb, int wf,
                                         int wmt, int l32, int h32, Acc& acc) {
  Ops o0, o1;
  read_ops(sa, sb, 0, wf, wmt, l32, h32, o0);
  read_ops(sa, sb, 1, wf, wmt, l32, h32, o1);
  mma(o0, acc);
  mma(o1, acc);
}

// Adapter slices of 32: acc[f][m] += sum_j Wl(f, j) * L[m][j] for j < r, Wl(f, j) at
// f*wl_fs + j*wl_js (elements), L [M, r] row-major, staged through slot 4.  Threads 0-255
// load feature row f0 + t, threads 256-511 token row m0 + t - 256.  A side whose rows are
// contiguous with r % 8 == 0 moves whole 16-byte chunks; otherwise element by element (any
// r, any stride: a transposed Wl such as A^T read straight from A [r, F] costs no extra
// launch, and its element loads are coalesced across the 256 feature threads).
__device__ __forceinline__ void adapter(const uint16_t* __restrict__ wl, int64_t wl_fs, int64_t wl_js, int64_t F,
                                        const uint16_t* __restrict__ Lm, int64_t M, int32_t r, int64_t f0, int64_t m0,
                                        int tid, int wf, int wmt, int l32, int h32, Acc& acc) {
  const bool wside = tid < 256;
  const int row = wside ? tid : tid - 256;
  const rsrc_t rw = make_rsrc(wl, (F - 1) * wl_fs * 2 + (int64_t)r * wl_js * 2);
  const rsrc_t rm = make_rsrc(Lm, M * (int64_t)r * 2);
  const bool vec = wside ? (wl_js == 1 && wl_fs == r && (r & 7) == 0) : ((r & 7) == 0);
  const int64_t f = f0 + row, m = m0 + row;
  const bool rok = wside ? f < F : m < M;
  const rsrc_t rr = wside ? rw : rm;
  const int64_t rowoff = (wside ? f : m) * (int64_t)r;  // vec: both sides are [rows, r]
  for (int32_t j0 = 0; j0 < r; j0 += BK) {
    uint4 c4[kChunks];
    if (vec) {
#pragma unroll
      for (int c = 0; c < kChunks; ++c) {
        const bool ok = rok && j0 + 8 * c < r;
        c4[c] = bload16(rr, ok ? (uint32_t)((rowoff + j0 + 8 * c) * 2) : kOOB);
      }
    } else {
      uint32_t e[BK];
      if (wside) {
#pragma unroll
        for (int q = 0; q < BK; ++q) {
          const bool ok = rok && j0 + q < r;
          e[q] = __builtin_amdgcn_raw_buffer_load_b16(rw, ok ? (int)((f * wl_fs + (int64_t)(j0 + q) * wl_js) * 2) : (int)kOOB, 0, 0);
        }
      } else {
#pragma unroll
        for (int q = 0; q < BK; ++q) {
          const bool ok = rok && j0 + q < r;
          e[q] = __builtin_amdgcn_raw_buffer_load_b16(rm, ok ? (int)((m * r + j0 + q) * 2) : (int)kOOB, 0, 0);
        }
      }
#pragma unroll
      for (int c = 0; c < kChunks; ++c)
        c4[c] = make_uint4((e[8 * c + 0] & 0xFFFFu) | (e[8 * c + 1] << 16), (e[8 * c + 2] & 0xFFFFu) | (e[8 * c + 3] << 16),
                           (e[8 * c + 4] & 0xFFFFu) | (e[8 * c + 5] << 16), (e[8 * c + 6] & 0xFFFFu) | (e[8 * c + 7] << 16));
    }
    uint4* dst = wside ? abuf<4>() : bbuf<4>();
    if (j0 > 0) lds_barrier();  // the previous slice's MFMA reads are done
#pragma unroll
    for (int c = 0; c < kChunks; ++c) dst[swz(row, c)] = c4[c];
    lds_barrier();
    mma_step(abuf<4>(), bbuf<4>(), wf, wmt, l32, h32, acc);
  }
}

// Epilogue.  C is [M, F] BF16 (token-major).  Register 4q + v of tile (i, j) holds feature
// 32 i + 8 q + 4 h32 + v of token 32 j + l32 within the wavefront's 128 x 64 tile.  The tile
// is staged in 16 KB of LDS as 64 token rows of 256 bytes (32 units of 8 bytes; unit u of
// row m at position u ^ (m & 31), so the 8-byte writes of 32 rows hit distinct banks), then
// read back 16 bytes per lane, 16 lanes per row, so every global store writes contiguous
// 256-byte row segments.  An odd row swizzle swaps the two 8-byte halves of a 16-byte read.
__device__ __forceinline__ uint4* epi_region(int wave) {
  switch (wave) {
    case 0: return s_a0;
    case 1: return s_a1;
    case 2: return s_a2;
    case 3: return s_a3;
    case 4: return s_a4;
    case 5: return s_b0;
    case 6: return s_b1;
    default: return s_b2;
  }
}
__device__ __forceinline__ void store_tile(uint16_t* __restrict__ C, int64_t M, int64_t F, int64_t f0, int64_t m0,
                                           int wave, int lane, int l32, int h32, const Acc& acc) {
  uint4* reg = epi_region(wave);
  uint2* reg2 = reinterpret_cast<uint2*>(reg);
#pragma unroll
  for (int j = 0; j < TJ; ++j) {
    const int m = 32 * j + l32;
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int u = 8 * i + 2 * q + h32;
        reg2[m * 32 + (u ^ (m & 31))] = make_uint2(pack_bf16x2(acc[i][j][4 * q + 0], acc[i][j][4 * q + 1]),
                                                   pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]));
      }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // this wavefront's LDS writes are done (it reads only its own region)
  const int c = lane & 15;
#pragma unroll
  for (int it = 0; it < 16; ++it) {
    const int m = 4 * it + (lane >> 4);
    const int s = m & 31;
    uint4 v = reg[m * 16 + (c ^ (s >> 1))];
    if (s & 1) v = make_uint4(v.z, v.w, v.x, v.y);
    const int64_t gm = m0 + m, gf = f0 + 8 * c;
    if (gm < M && gf < F) *reinterpret_cast<uint4*>(C + gm * F + gf) = v;
  }
}

// FP32 partial of a split: the wavefront's 128 features x 64 tokens go out in two passes of
// 32 tokens (16 KB of its staging region: 32 rows of 512 bytes, 16-byte unit u of row m at
// u ^ (m & 31)), read back 32 lanes per row so that each store writes two 512-byte row
// segments.  Register 4q + v of tile (i, j) holds feature 32 i + 8 q + 4 h32 + v.
__device__ __forceinline__ void store_part(float* __restrict__ P, int64_t M, int64_t F, int64_t f0, int64_t m0,
                                           int wave, int lane, int l32, int h32, const Acc& acc) {
  uint4* reg = epi_region(wave);
#pragma unroll
  for (int j = 0; j < TJ; ++j) {
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int u = 8 * i + 2 * q + h32;
        reg[l32 * 32 + (u ^ l32)] = make_uint4(__float_as_uint(acc[i][j][4 * q + 0]), __float_as_uint(acc[i][j][4 * q + 1]),
                                               __float_as_uint(acc[i][j][4 * q + 2]), __float_as_uint(acc[i][j][4 * q + 3]));
      }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // this wavefront's LDS writes are done (it reads only its own region)
    const int c = lane & 31;
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      const int m = 2 * it + (lane >> 5);
      const uint4 v = reg[m * 32 + (c ^ m)];
      const int64_t gm = m0 + 32 * j + m, gf = f0 + 4 * c;
      if (gm < M && gf < F) *reinterpret_cast<uint4*>(P + gm * F + gf) = v;
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // reads done before the next pass rewrites the region
  }
}

// C [M, F] = bf16(sum over s of P[s] [M, F]), the splits added in order s = 0, 1, ...; one
// thread per 8 consecutive features (F % 16 == 0).
__global__ __launch_bounds__(256) void k_sum_parts(const float* __restrict__ P, int32_t ks, int64_t M, int64_t F,
                                                   uint16_t* __restrict__ C) {
  const int64_t n8 = M * F / 8;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += stride) {
    float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int32_t sp = 0; sp < ks; ++sp) {
      const float4* src = reinterpret_cast<const float4*>(P + (int64_t)sp * M * F) + 2 * i;
      const float4 x = src[0], y = src[1];
      a[0] += x.x; a[1] += x.y; a[2] += x.z; a[3] += x.w;
      a[4] += y.x; a[5] += y.y; a[6] += y.z; a[7] += y.w;
    }
    reinterpret_cast<uint4*>(C)[i] = make_uint4(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]),
                                                 pack_bf16x2(a[4], a[5]), pack_bf16x2(a[6], a[7]));
  }
}

// Consecutive workgroups are dealt round-robin to the 8 XCDs (each with its own L2):
// renumber so that one XCD gets a compact block of tiles.
// - When the feature tiles divide into columns of 4 that split the grid into 8 equal blocks
//   (4 feature tiles x n/32 token tiles; up to 32 feature tiles), each XCD takes one block:
//   at 16 x 16 tiles its L2 then sees 4 weight row blocks and 8 token row blocks per
//   reduction step instead of 16 and 2.
// - Wider products (feature tiles a multiple of 8, more than 32 of them) give each XCD its
//   own gx/8 feature columns over all token tiles, walked in bands of bw columns (the largest
//   divisor of gx/8 up to 8), columns fastest: each weight row block then goes to one XCD
//   only, and the 32 workgroups an XCD runs at once cover about bw columns x 32/bw token
//   tiles.  Taking runs in feature-fastest order instead sent every weight row block to all
//   8 XCDs (28672 x 8192 at M = 2048: 4.97 GB fetched from beyond the L2s per launch).
// - Otherwise each XCD takes a run in feature-fastest order.
__device__ __forceinline__ void tile_xy(int64_t& tx, int64_t& ty) {
  const uint32_t gx = gridDim.x, gy = gridDim.y, n = gridDim.x * gridDim.y;
  uint32_t L = blockIdx.x + gx * blockIdx.y;
  if ((n & 31) == 0 && gx % 4 == 0 && 32 % gx == 0) {
    L = (L & 7) * (n >> 3) + (L >> 3);
    const uint32_t per = n >> 3, xcd = L / per, w = L % per, cols = gx / 4;
    tx = (xcd % cols) * 4 + (w % 4);
    ty = (xcd / cols) * (per / 4) + w / 4;
    return;
  }
  if (gx % 8 == 0) {
    const uint32_t xcd = L & 7, idx = L >> 3, cx = gx >> 3;
    uint32_t bw = 1;
    for (uint32_t d = 8; d > 1; --d)
      if (cx % d == 0) {
        bw = d;
        break;
      }
    const uint32_t band = idx / (bw * gy), r = idx % (bw * gy);
    tx = xcd * cx + band * bw + r % bw;
    ty = r / bw;
    return;
  }
  if ((n & 7) == 0) L = (L & 7) * (n >> 3) + (L >> 3);
  tx = L % gx;
  ty = L / gx;
}

// Ring step kb in slot S = kb % 5.  Steps run in pairs (2t, 2t+1) between barriers: the
// barrier after step 2t+1 publishes the slots of steps 2t+2 and 2t+3 and retires those of
// steps up to 2t+1, so within a pair the wavefronts of a SIMD may drift apart and fill each
// other's gaps on the matrix pipe.  Step kb issues the loads of step kb+3 into the slot of
// step kb-2, which every wavefront finished reading before the last barrier.  The last three
// steps issue them too, for steps past the range: those read zeros (or the next split's
// columns) into slots that are never read again, and the epilogue waits for them.  A branch
// around each load cost more than the loads (about 2% of the launch).
//
// The second half (ks = 1) of the previous step's MFMAs is deferred: its operands are in
// `o1`, so those MFMAs run while this step's operand reads are in flight.  The four ring
// loads are issued one at a time between groups of four MFMAs: a CU's address unit takes
// one 1 KB load per ~16 clocks, and a burst at the top of the step would stall every
// wavefront's (in-order) issue behind it.
template <int S, bool ODD, bool FULLK>
__device__ __forceinline__ void nt_step(const Ring& ra, const Ring& rb, uint32_t kb, uint32_t nk, int wf, int wmt,
                                        int l32, int h32, Ops& o1, Acc& acc) {
  uint4* const na = abuf<(S + 3) % kRing>();
  uint4* const nb = bbuf<(S + 3) % kRing>();
  Ops o0;
  read_ops(abuf<S>(), bbuf<S>(), 0, wf, wmt, l32, h32, o0);
  mma_half(o1, 0, acc);  // ks = 1 of step kb - 1
  __builtin_amdgcn_sched_barrier(0);
  ra.issue1<FULLK>(na, kb + 3, 0);
  __builtin_amdgcn_sched_barrier(0);
  mma_half(o1, 1, acc);
  __builtin_amdgcn_sched_barrier(0);
  ra.issue1<FULLK>(na, kb + 3, 1);
  __builtin_amdgcn_sched_barrier(0);
  read_ops(abuf<S>(), bbuf<S>(), 1, wf, wmt, l32, h32, o1);
  mma_half(o0, 0, acc);
  __builtin_amdgcn_sched_barrier(0);
  rb.issue1<FULLK>(nb, kb + 3, 0);
  __builtin_amdgcn_sched_barrier(0);
  mma_half(o0, 1, acc);
  __builtin_amdgcn_sched_barrier(0);
  rb.issue1<FULLK>(nb, kb + 3, 1);
  if (ODD) {
    wait_vm<4>();  // this wavefront's loads of steps kb+1 and kb+2 are complete (kb+3's may be pending)
    lds_barrier();
  }
}

template <bool SPLIT, bool FULLK>
__global__ __launch_bounds__(kThreads, 1) void k_gemm_nt(const uint16_t* __restrict__ A, int64_t F,
                                                         const uint16_t* __restrict__ B, int64_t M, int64_t Kr,
                                                         const uint16_t* __restrict__ wl, int64_t wl_fs,
                                                         int64_t wl_js, const uint16_t* __restrict__ Lm, int32_t r,
                                                         uint16_t* __restrict__ C, float* __restrict__ part,
                                                         uint32_t kb_per) {
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, h32 = lane >> 5;
  const int wf = (wave & 1) * 128, wmt = (wave >> 1) * 64;
  int64_t tx, ty;
  tile_xy(tx, ty);
  const int64_t f0 = tx * BF, m0 = ty * BMT;
  const uint32_t nk_all = (uint32_t)((Kr + BK - 1) / BK);
  // this workgroup's reduction steps: [kb0, kb0 + nk)
  const uint32_t kb0 = SPLIT ? blockIdx.z * kb_per : 0u;
  const uint32_t nk = SPLIT ? (kb0 + kb_per <= nk_all ? kb_per : (kb0 < nk_all ? nk_all - kb0 : 0u)) : nk_all;

  Ring ra, rb;
  ra.init<FULLK>(A, F, f0, Kr, wave, lane, kb0);
  rb.init<FULLK>(B, M, m0, Kr, wave, lane, kb0);
  // steps 0..2 in flight while the adapter slices run through slot 4
  ra.issue<FULLK>(abuf<0>(), 0);
  rb.issue<FULLK>(bbuf<0>(), 0);
  if (nk > 1) {
    ra.issue<FULLK>(abuf<1>(), 1);
    rb.issue<FULLK>(bbuf<1>(), 1);
  }
  if (nk > 2) {
    ra.issue<FULLK>(abuf<2>(), 2);
    rb.issue<FULLK>(bbuf<2>(), 2);
  }
  Acc acc;
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = f32x16_t{};
  if (!SPLIT || blockIdx.z == 0) adapter(wl, wl_fs, wl_js, F, Lm, M, r, f0, m0, tid, wf, wmt, l32, h32, acc);
  wait_vm<0>();
  lds_barrier();  // steps 0, 1 landed everywhere; the adapter's reads of slot 4 are done

  Ops o1;  // deferred second half of the previous step: none before step 0
#pragma unroll
  for (int i = 0; i < TI; ++i) o1.a[i] = bf16x8_t{};
#pragma unroll
  for (int j = 0; j < TJ; ++j) o1.b[j] = bf16x8_t{};
  for (uint32_t kb = 0; kb < nk; kb += 10) {
    nt_step<0, false, FULLK>(ra, rb, kb + 0, nk, wf, wmt, l32, h32, o1, acc);
    if (kb + 1 >= nk) break;
    nt_step<1, true, FULLK>(ra, rb, kb + 1, nk, wf, wmt, l32, h32, o1, acc);
    if (kb + 2 >= nk) break;
    nt_step<2, false, FULLK>(ra, rb, kb + 2, nk, wf, wmt, l32, h32, o1, acc);
    if (kb + 3 >= nk) break;
    nt_step<3, true, FULLK>(ra, rb, kb + 3, nk, wf, wmt, l32, h32, o1, acc);
    if (kb + 4 >= nk) break;
    nt_step<4, false, FULLK>(ra, rb, kb + 4, nk, wf, wmt, l32, h32, o1, acc);
    if (kb + 5 >= nk) break;
    nt_step<0, true, FULLK>(ra, rb, kb + 5, nk, wf, wmt, l32, h32, o1, acc);
    if (kb + 6 >= nk) break;
    nt_step<1, false, FULLK>(ra, rb, kb + 6, nk, wf, wmt, l32, h32, o1, acc);
    if (kb + 7 >= nk) break;
    nt_step<2, true, FULLK>(ra, rb, kb + 7, nk, wf, wmt, l32, h32, o1, acc);
    if (kb + 8 >= nk) break;
    nt_step<3, false, FULLK>(ra, rb, kb + 8, nk, wf, wmt, l32, h32, o1, acc);
    if (kb + 9 >= nk) break;
    nt_step<4, true, FULLK>(ra, rb, kb + 9, nk, wf, wmt, l32, h32, o1, acc);
  }
  mma(o1, acc);  // ks = 1 of the last step
  wait_vm<0>();   // the loads issued past the range have landed
  lds_barrier();  // every wavefront is done with the ring slots, which now stage the epilogue
  if (SPLIT)
    store_part(part + (int64_t)blockIdx.z * M * F, M, F, f0 + wf, m0 + wmt, wave, lane, l32, h32, acc);
  else
    store_tile(C, M, F, f0 + wf, m0 + wmt, wave, lane, l32, h32, acc);
}

}  // namespace

int32_t gemm_nt_ksplit(int64_t F, int64_t M, int64_t Kr) {
  const int64_t tiles = ((F + BF - 1) / BF) * ((M + BMT - 1) / BMT);
  const int64_t nk = (Kr + BK - 1) / BK;
  if (tiles > 128) return 1;
  int64_t ks = 256 / tiles;
  if (ks > nk / 16) ks = nk / 16;  // at least 16 reduction steps per split
  return ks >= 2 ? (int32_t)ks : 1;
}

hipError_t launch_gemm_nt(const uint16_t* A, int64_t F, const uint16_t* B, int64_t M, int64_t Kr,
                          const uint16_t* wl, int64_t wl_fs, int64_t wl_js, const uint16_t* L, int32_t r,
                          uint16_t* C, int kernel_id, hipStream_t st, float* part, int32_t ksplit) {
  const int64_t nk = (Kr + BK - 1) / BK;
  if (ksplit > 1 && (!part || F % 16 != 0)) return hipErrorInvalidValue;
  const uint32_t kb_per = ksplit > 1 ? (uint32_t)((nk + ksplit - 1) / ksplit) : (uint32_t)nk;
  dim3 grid((unsigned)((F + BF - 1) / BF), (unsigned)((M + BMT - 1) / BMT), (unsigned)(ksplit > 1 ? ksplit : 1));
  LaunchTimer t(kernel_id, st);
  const bool fullk = Kr % BK == 0;
#define GEMM_ARGS A, F, B, M, Kr, wl, wl_fs, wl_js, L, r, C, part, kb_per
  if (ksplit > 1 && fullk)
    hipExtLaunchKernelGGL(k_gemm_nt<true, true>, grid, dim3(kThreads), 0, st, t.start, t.stop, 0, GEMM_ARGS);
  else if (ksplit > 1)
    hipExtLaunchKernelGGL(k_gemm_nt<true, false>, grid, dim3(kThreads), 0, st, t.start, t.stop, 0, GEMM_ARGS);
  else if (fullk)
    hipExtLaunchKernelGGL(k_gemm_nt<false, true>, grid, dim3(kThreads), 0, st, t.start, t.stop, 0, GEMM_ARGS);
  else
    hipExtLaunchKernelGGL(k_gemm_nt<false, false>, grid, dim3(kThreads), 0, st, t.start, t.stop, 0, GEMM_ARGS);
#undef GEMM_ARGS
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || ksplit <= 1) return e;
  const int64_t n8 = M * F / 8;
  const int64_t blocks = std::min<int64_t>((n8 + 255) / 256, 2048);
  hipLaunchKernelGGL(k_sum_parts, dim3((unsigned)blocks), dim3(256), 0, st, part, ksplit, M, F, C);
  return hipGetLastError();
}

}  // namespace qlora
