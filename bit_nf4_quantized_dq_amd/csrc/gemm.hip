// Fused dequantize -> BF16 MFMA GEMMs for many tokens (M > 16).
//
// "QLoRA: Quantize Base Weights to 4-Bit", Section 3: the 4-bit weights stay in HBM; a
// tile is expanded to BF16 on chip and fed to the matrix units, and the adapter branch is
// added.  "QLoRA -- Fine-Tuning a 65B Model on One GPU", "Where the gradients actually go":
// the input gradient runs through the dequantized weights (dX = dY w_hat + s G A).
//
// Both kernels compute an output tile D[f][m] (f = output feature, m = token) with MFMA
// 32x32x16 BF16: the decoded weights are the A operand (rows f), activations the B operand
// (columns m).
//
//   forward : f = n (d_out), reduction over k (d_in).  W rows are k-contiguous, so a thread
//             decodes one (row, 64-block) = 8 code words with a per-block scaled BF16 table
//             (bit-exact w_hat) and writes 8 16-byte chunks of LDS row f.
//   dX      : f = k (d_in), reduction over n (d_out).  The quantization blocks now run along
//             the output dimension, so a thread decodes 8 rows x 8 columns with the unscaled
//             table, applies each row's constant in FP32 (bit-exact as well), and writes the
//             8 x 8 tile transposed (8 n-values per feature k).  The 8 lanes that share a
//             block column each fetch one row's constant and pass it on with lane swizzles.
// Adapter term: ceil(r/32) extra reduction steps of width 32 multiply the prescaled BF16
// side input (s T for forward, s G for dX) by B (forward) or A^T (dX); they run first, so
// the accumulators start from the adapter term.
//
// Tiling: 256 (features) x 256 (tokens) per workgroup, reduction step 64, 8 wavefronts
// (two per SIMD) in a 2 x 4 grid of 128 x 64 wavefront tiles (4 x 2 MFMA tiles, 128 FP32
// accumulators per lane).  Pipeline, per reduction step kb:
//   * every wavefront issues direct buffer->LDS loads of the activation tile of step kb+2
//     into a three-slot LDS ring (no registers held while the loads are in flight);
//   * wavefronts 0-3 issue the code loads of step kb+2 (forward) or kb+1 (dX, whose
//     per-step register set is larger) into registers;
//   * all wavefronts run the MFMAs of step kb from LDS;
//   * wavefronts 0-3 decode the codes of step kb+1 into the other weight buffer;
//   * each wavefront waits for its own ring loads of step kb+1, then one barrier.
// The step loop is unrolled six times so that every LDS buffer index is a compile-time
// constant: the compiler then waits only for the ring slot an access touches.  Global
// loads are raw buffer loads (zero outside the tensor, also into LDS), so ragged tiles need
// no branches in the loop.  16-byte LDS chunks are XOR-swizzled by row; the ring loads pick
// their global chunk so that each lane's 16 bytes land in the swizzled slot.
#include "qlora_device.h"
#include "qlora_host.h"

namespace qlora {
namespace {

constexpr int kThreads = 512;
constexpr int kStage = 256;          // threads that decode weights (wavefronts 0-3)
constexpr int BF = 256;              // features per tile
constexpr int BMT = 256;             // tokens per tile
constexpr int BK = 64;               // reduction step
constexpr int kChunks = BK / 8;      // 16-byte chunks per LDS row
constexpr int kTile = 256 * kChunks; // 16-byte chunks per LDS tile
constexpr int TI = 4, TJ = 2;        // 32x32 MFMA tiles per wavefront: 128 features x 64 tokens
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef f32x16_t Acc[TI][TJ];
typedef __attribute__((address_space(3))) void lds_void;

// Decoded weight tiles (double buffer) and the activation ring: 5 x 32 KB = 160 KB.
__shared__ uint4 s_w0[kTile], s_w1[kTile];
__shared__ uint4 s_x0[kTile], s_x1[kTile], s_x2[kTile];

template <int I> __device__ __forceinline__ uint4* wbuf() { return I == 0 ? s_w0 : s_w1; }
template <int I> __device__ __forceinline__ uint4* xbuf() { return I == 0 ? s_x0 : (I == 1 ? s_x1 : s_x2); }

__device__ __forceinline__ f32x16_t mfma32(const bf16x8_t& a, const bf16x8_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kChunks + (chunk ^ ((row ^ (row >> 3)) & 7));
}

// s_waitcnt with only the vector-memory counter limited to N (LDS counter untouched).
template <int N> __device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}
// Own LDS writes done, then the workgroup barrier.  The asm statement is also a compiler
// barrier for memory accesses; the vector-memory waits that the ring needs are explicit.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("s_barrier" ::: "memory");
}

// ---- activation ring: rows = tokens (from m0), columns = reduction index (Kr in total).
// Wavefront w fills rows 32w .. 32w+31 of a stage with 4 loads of 8 rows x 8 chunks; lane p
// of load j writes chunk slot (p & 7) of row 8(4w+j) + (p >> 3) and therefore fetches the
// logical chunk that the swizzle maps to that slot.
struct ActRing {
  rsrc_t r;
  uint32_t base[4];  // byte offset of the lane's chunk at reduction index 0; kOOB past M
  uint32_t col[4];   // the lane's first reduction index within a step
  uint32_t Kr;
  int wave;

  __device__ __forceinline__ void init(const uint16_t* A, int64_t M, int64_t m0, int64_t Kr_, int w, int lane) {
    const int64_t rows = M - m0 < BMT ? M - m0 : BMT;
    r = make_rsrc(A + m0 * Kr_, rows * Kr_ * 2);
    Kr = (uint32_t)Kr_;
    wave = w;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = 8 * (4 * w + j) + (lane >> 3);
      const int lc = (lane & 7) ^ ((row ^ (row >> 3)) & 7);
      col[j] = 8 * lc;
      base[j] = row < rows ? (uint32_t)(row * Kr_ * 2 + 16 * lc) : kOOB;
    }
  }
  template <int SLOT> __device__ __forceinline__ void issue(uint32_t kb) const {
    const uint32_t k0 = kb * BK;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t off = (base[j] != kOOB && k0 + col[j] < Kr) ? base[j] + 2 * k0 : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(xbuf<SLOT>() + (4 * wave + j) * 64), 16, off, 0, 0, 0);
    }
  }
};

// ---- forward weight tile: thread t decodes row f0 + t, block kb (64 weights)
struct FwdDec {
  static constexpr int kLoads = 4;  // vector-memory instructions per load()
  static constexpr int kDist = 2;   // steps between the code loads and their decode
  struct Regs {
    uint4 c0, c1;
    uint32_t c8, c2;
  };
  rsrc_t codes;  // from row f0
  rsrc_t code8;  // from block f0 * nb_row
  rsrc_t c2s;    // whole tensor
  uint32_t row_off;  // t * K / 2
  uint32_t blk;      // t * nb_row (local block index of the row's first block)
  uint32_t blk0;     // f0 * nb_row
  float mu;
  Nf4Tables T;
  int t;

  __device__ __forceinline__ void load(Regs& R, uint32_t kb) const {
    R.c0 = bload16(codes, row_off + kb * 32);
    R.c1 = bload16(codes, row_off + kb * 32 + 16);
    R.c8 = bload1(code8, blk + kb);
    R.c2 = bload4(c2s, ((blk0 + blk + kb) >> 8) * 4);
  }
  __device__ __forceinline__ void store(uint4* __restrict__ s, const Regs& R, uint32_t) const {
    Lut L;
    build_scaled_lut(T, block_scale(R.c8, __uint_as_float(R.c2), mu), L);
    const uint32_t words[8] = {R.c0.x, R.c0.y, R.c0.z, R.c0.w, R.c1.x, R.c1.y, R.c1.z, R.c1.w};
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      uint32_t o[4];
      decode8(words[c], L, o);
      s[swz(t, c)] = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
};

// Value of lane I of the lane's aligned group of 8 (swizzle and-mask 0x18, or-mask I).
template <int I> __device__ __forceinline__ float bcast8(int v) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(v, 0x18 | (I << 5)));
}

// ---- dX weight tile: thread t decodes rows n0 + 8*(t>>5) + i (i < 8) at columns
// k0 + 8*(t&31) + e (e < 8), one code word per row.  Lane e of each aligned group of 8 lanes
// fetches the block constant of row n0 + 8*(t>>5) + e.
struct DxDec {
  static constexpr int kLoads = 10;
  static constexpr int kDist = 1;
  struct Regs {
    uint32_t w[8];
    uint32_t c8, c2;
  };
  const uint8_t* codes;  // whole tensor (the descriptor is rebased per step)
  int64_t codes_bytes;
  rsrc_t code8, c2s;     // whole tensor
  uint32_t code_off;  // row 8*rg, column k0 + 8*kc; kOOB when past K
  uint32_t row_bytes; // K / 2
  uint32_t nb_row;    // K / 64
  uint32_t blk_off;   // block index of row 8*rg + e at the block column of k0 + 8*kc
  uint32_t N;
  uint32_t own_row;   // 8*rg + e
  float mu;
  Lut L;
  int t;

  __device__ __forceinline__ void load(Regs& R, uint32_t kb) const {
    const uint32_t n0 = kb * BK;
    const bool kok = code_off != kOOB;
    // descriptor based at row n0 (wave-uniform), so the per-lane offsets stay loop-invariant
    const int64_t step = (int64_t)n0 * row_bytes;
    const rsrc_t rc = make_rsrc(codes + step, codes_bytes - step);
#pragma unroll
    for (int i = 0; i < 8; ++i) R.w[i] = bload4(rc, kok ? code_off + i * row_bytes : kOOB);
    const bool ok = kok && n0 + own_row < N;
    const uint32_t b = blk_off + n0 * nb_row;
    R.c8 = bload1(code8, ok ? b : kOOB);
    R.c2 = bload4(c2s, ok ? (b >> 8) * 4 : kOOB);
  }
  __device__ __forceinline__ void store(uint4* __restrict__ s, const Regs& R, uint32_t kb) const {
    // rows past N: codes read as 0 and the constant is forced to 0, so the tile is +-0
    const bool ok = kb * BK + own_row < N;
    const float own = ok ? block_scale(R.c8, __uint_as_float(R.c2), mu) : 0.f;
    const int ownb = __float_as_int(own);
    const float sc[8] = {bcast8<0>(ownb), bcast8<1>(ownb), bcast8<2>(ownb), bcast8<3>(ownb),
                         bcast8<4>(ownb), bcast8<5>(ownb), bcast8<6>(ownb), bcast8<7>(ownb)};
    const int rg = t >> 5, kc = t & 31;
    uint2* s2 = reinterpret_cast<uint2*>(s);
    // two halves of 4 rows each (8-byte LDS writes) keep the live transposed block small
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t o[8][2];  // o[e][q]: BF16 pair (rows 4h+2q, 4h+2q+1) of column e
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int p = 2 * h + q;
        uint32_t da[4], db[4];
        decode8(R.w[2 * p], L, da);
        decode8(R.w[2 * p + 1], L, db);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t a = da[e >> 1], b = db[e >> 1];
          const float fa = (e & 1) ? bf16hi_to_f32(a) : bf16lo_to_f32(a);
          const float fb = (e & 1) ? bf16hi_to_f32(b) : bf16lo_to_f32(b);
          o[e][q] = pack_bf16x2(fa * sc[2 * p], fb * sc[2 * p + 1]);
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) s2[2 * swz(8 * kc + e, rg) + h] = make_uint2(o[e][0], o[e][1]);
    }
  }
};

// ---- MFMA operand addressing.  Operand rows are base + 32 i + l32 with base a multiple of
// 64, so the swizzle term (row ^ (row >> 3)) & 7 equals (l32 & 7) ^ (l32 >> 3) ^ 4 (i & 1),
// and the chunk of 16-wide reduction step ks, (2 ks + h32) ^ swizzle, is
// (2 ks ^ 4 (i & 1)) ^ g with the per-lane g = h32 ^ (l32 & 7) ^ (l32 >> 3).  Written this
// way the compiler keeps four per-lane bases and folds the rest into immediate offsets.
__device__ __forceinline__ int op_lane(int l32, int h32) { return h32 ^ (l32 & 7) ^ (l32 >> 3); }
__device__ __forceinline__ int op_idx(int base, int i, int ks, int l32, int g) {
  return (base + 32 * i + l32) * kChunks + ((2 * ks ^ 4 * (i & 1)) ^ g);
}

// ---- MFMA on one LDS stage: four 16-wide reduction steps.  Lane l supplies row (l & 31) of
// each operand tile and the 8 reduction indices 8*(l >> 5) of the step.  Operands are read
// one 16-wide step at a time; the other wavefront on the SIMD covers the LDS latency.
__device__ __forceinline__ void mma_stage(const uint4* __restrict__ sw, const uint4* __restrict__ sx,
                                          int wf, int wmt, int l32, int g, Acc& acc) {
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    bf16x8_t a[TI], b[TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i) a[i] = as_bf16x8(sw[op_idx(wf, i, ks, l32, g)]);
#pragma unroll
    for (int j = 0; j < TJ; ++j) b[j] = as_bf16x8(sx[op_idx(wmt, j, ks, l32, g)]);
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) acc[i][j] = mfma32(a[i], b[j], acc[i][j]);
  }
}

// Adapter K-slices: acc[f][m] += sum_j wl[f, j] * Lm[m, j] for j < r, in slices of 32 staged
// through LDS (weights side: W-role threads, one feature row each; tokens side: the others).
// wl element (f, j) sits at f * wl_fs + j * wl_js (elements); Lm is [M, r] row-major.
__device__ __forceinline__ void lora_slices(const uint16_t* __restrict__ wl, int64_t wl_fs, int64_t wl_js,
                                            int64_t F, const uint16_t* __restrict__ Lm, int64_t M,
                                            int32_t r, int64_t f0, int64_t m0, bool wrole, int st,
                                            uint4* __restrict__ sw, uint4* __restrict__ sx, int wf,
                                            int wmt, int lr, int lg, Acc& acc) {
  const rsrc_t rw = make_rsrc(wl, (F - 1) * wl_fs * 2 + (int64_t)r * wl_js * 2);
  const rsrc_t rm = make_rsrc(Lm, M * (int64_t)r * 2);
  for (int32_t j0 = 0; j0 < r; j0 += 32) {
    uint32_t e[32];
    if (wrole) {
      const int64_t f = f0 + st;
#pragma unroll
      for (int q = 0; q < 32; ++q) {
        const bool ok = f < F && j0 + q < r;
        e[q] = __builtin_amdgcn_raw_buffer_load_b16(rw, ok ? (int)((f * wl_fs + (int64_t)(j0 + q) * wl_js) * 2) : (int)kOOB, 0, 0);
      }
    } else {
      const int64_t m = m0 + st;
#pragma unroll
      for (int q = 0; q < 32; ++q) {
        const bool ok = m < M && j0 + q < r;
        e[q] = __builtin_amdgcn_raw_buffer_load_b16(rm, ok ? (int)((m * r + j0 + q) * 2) : (int)kOOB, 0, 0);
      }
    }
    __syncthreads();  // previous slice's reads are done
    uint4* dst = wrole ? sw : sx;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      dst[swz(st, c)] = make_uint4((e[8 * c + 0] & 0xFFFFu) | (e[8 * c + 1] << 16), (e[8 * c + 2] & 0xFFFFu) | (e[8 * c + 3] << 16),
                                   (e[8 * c + 4] & 0xFFFFu) | (e[8 * c + 5] << 16), (e[8 * c + 6] & 0xFFFFu) | (e[8 * c + 7] << 16));
    }
    __syncthreads();
    const int g = op_lane(lr, lg);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8_t a[TI], b[TJ];
#pragma unroll
      for (int i = 0; i < TI; ++i) a[i] = as_bf16x8(sw[op_idx(wf, i, ks, lr, g)]);
#pragma unroll
      for (int j = 0; j < TJ; ++j) b[j] = as_bf16x8(sx[op_idx(wmt, j, ks, lr, g)]);
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) acc[i][j] = mfma32(a[i], b[j], acc[i][j]);
    }
  }
}

// Store D[f][m] tile (32x32 layout): register 4q + v of tile (i, j) holds feature
// f = f0 + 32 i + 8 q + 4 h32 + v of token m = m0 + 32 j + l32.
__device__ __forceinline__ void store_tile(uint16_t* __restrict__ Y, int64_t M, int64_t F, int64_t f0,
                                           int64_t m0, int l32, int h32, const Acc& acc) {
#pragma unroll
  for (int j = 0; j < TJ; ++j) {
    const int64_t m = m0 + 32 * j + l32;
    if (m >= M) continue;
#pragma unroll
    for (int i = 0; i < TI; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t f = f0 + 32 * i + 8 * q + 4 * h32;
        if (f < F) {
          const uint32_t lo = pack_bf16x2(acc[i][j][4 * q + 0], acc[i][j][4 * q + 1]);
          const uint32_t hi = pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
          *reinterpret_cast<uint2*>(Y + m * F + f) = make_uint2(lo, hi);
        }
      }
    }
  }
}

__device__ __forceinline__ void zero_acc(Acc& acc) {
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = f32x16_t{};
}

// Tile coordinates: consecutive workgroups are dealt round-robin to the 8 XCDs (each with
// its own L2), so renumber them such that one XCD receives a contiguous run of tiles in
// feature-fastest order -- a few token rows of tiles per XCD, sharing their activations.
__device__ __forceinline__ void tile_xy(int64_t& tx, int64_t& ty) {
  const uint32_t gx = gridDim.x, n = gridDim.x * gridDim.y;
  uint32_t L = blockIdx.x + gx * blockIdx.y;
  if ((n & 7) == 0) L = (L & 7) * (n >> 3) + (L >> 3);
  tx = L % gx;
  ty = L / gx;
}

// One reduction step (the pipeline described at the top); XS / WB are the ring slot and
// weight buffer of step kb, known at compile time.  With Dec::kDist == 2 the codes of step
// kb+1 were loaded one step earlier (into `cur`) and those of kb+2 are loaded now (into
// `nxt`); with kDist == 1 the codes of step kb+1 are loaded at the start of this step (into
// `cur`), before the ring loads, so their decode does not wait for the ring.
template <int XS, int WB, class Dec>
__device__ __forceinline__ void gemm_step(const Dec& dec, const ActRing& ring, uint32_t kb, uint32_t nk,
                                          typename Dec::Regs& cur, typename Dec::Regs& nxt, bool wrole,
                                          int wf, int wmt, int l32, int h32, Acc& acc) {
  const bool has1 = kb + 1 < nk, has2 = kb + 2 < nk;
  if (Dec::kDist == 1 && has1 && wrole) dec.load(cur, kb + 1);
  if (has2) {
    ring.template issue<(XS + 2) % 3>(kb + 2);
    if (Dec::kDist == 2 && wrole) dec.load(nxt, kb + 2);
  }
  mma_stage(wbuf<WB>(), xbuf<XS>(), wf, wmt, l32, op_lane(l32, h32), acc);
  // keep the decode's temporaries out of the MFMA phase (they would not fit beside it)
  __builtin_amdgcn_sched_barrier(0);
  if (has1 && wrole) dec.store(wbuf<WB ^ 1>(), cur, kb + 1);
  // this wavefront's ring loads of step kb+1 are complete (only step kb+2's may be pending)
  if (has2) {
    if (Dec::kDist == 2 && wrole) wait_vm<4 + Dec::kLoads>();
    else wait_vm<4>();
  } else {
    wait_vm<0>();
  }
  lds_barrier();
}

// Steps 0 .. nk-1; with kDist == 2, step kb decodes from regs[(kb+1)&1] and loads step kb+2
// into regs[kb&1]; with kDist == 1 the same register roles apply to the step's own load.
template <class Dec>
__device__ __forceinline__ void gemm_main(const Dec& dec, const ActRing& ring, uint32_t nk, bool wrole,
                                          int wf, int wmt, int l32, int h32, typename Dec::Regs& r0,
                                          typename Dec::Regs& r1, Acc& acc) {
  for (uint32_t kb = 0; kb < nk; kb += 6) {
    gemm_step<0, 0>(dec, ring, kb + 0, nk, r1, r0, wrole, wf, wmt, l32, h32, acc);
    if (kb + 1 >= nk) break;
    gemm_step<1, 1>(dec, ring, kb + 1, nk, r0, r1, wrole, wf, wmt, l32, h32, acc);
    if (kb + 2 >= nk) break;
    gemm_step<2, 0>(dec, ring, kb + 2, nk, r1, r0, wrole, wf, wmt, l32, h32, acc);
    if (kb + 3 >= nk) break;
    gemm_step<0, 1>(dec, ring, kb + 3, nk, r0, r1, wrole, wf, wmt, l32, h32, acc);
    if (kb + 4 >= nk) break;
    gemm_step<1, 0>(dec, ring, kb + 4, nk, r1, r0, wrole, wf, wmt, l32, h32, acc);
    if (kb + 5 >= nk) break;
    gemm_step<2, 1>(dec, ring, kb + 5, nk, r0, r1, wrole, wf, wmt, l32, h32, acc);
  }
}

// Prologue: ring and code loads of steps 0 and 1, the adapter slices (through the weight
// buffer of step 1 and the ring slot of step 2), decode of step 0, one barrier.
template <class Dec>
__device__ __forceinline__ void gemm_prologue(const Dec& dec, const ActRing& ring, uint32_t nk, bool wrole,
                                              typename Dec::Regs& r0, typename Dec::Regs& r1,
                                              const uint16_t* wl, int64_t wl_fs, int64_t wl_js, int64_t F,
                                              const uint16_t* Lm, int64_t M, int32_t r, int64_t f0,
                                              int64_t m0, int st, int wf, int wmt, int l32, int h32,
                                              Acc& acc) {
  ring.template issue<0>(0);
  if (wrole) dec.load(r0, 0);
  if (nk > 1) {
    ring.template issue<1>(1);
    if (Dec::kDist == 2 && wrole) dec.load(r1, 1);
  }
  zero_acc(acc);
  lora_slices(wl, wl_fs, wl_js, F, Lm, M, r, f0, m0, wrole, st, s_w1, s_x2, wf, wmt, l32, h32, acc);
  if (wrole) dec.store(s_w0, r0, 0);
  wait_vm<0>();
  lds_barrier();  // also: the adapter slices' reads of s_w1 / s_x2 are done
}

__global__ __launch_bounds__(kThreads, 1) void k_gemm_fwd(
    const uint32_t* __restrict__ codes, const uint8_t* __restrict__ code8,
    const float* __restrict__ c2s, const float* __restrict__ mu_p, int64_t N, int64_t K,
    const uint16_t* __restrict__ X, int64_t M, const uint16_t* __restrict__ Lm,
    const uint16_t* __restrict__ Bl, int32_t r, uint16_t* __restrict__ Y, Nf4Tables T) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h32 = lane >> 5;
  const int wf = (wave & 1) * 128, wmt = (wave >> 1) * 64;
  const bool wrole = tid < kStage;
  const int st = wrole ? tid : tid - kStage;
  int64_t tx, ty;
  tile_xy(tx, ty);
  const int64_t f0 = tx * BF, m0 = ty * BMT;
  const uint32_t nk = (uint32_t)(K / BK);

  ActRing ring;
  ring.init(X, M, m0, K, wave, lane);
  FwdDec dec;
  dec.codes = make_rsrc(reinterpret_cast<const uint8_t*>(codes) + f0 * (K / 2), (N - f0) * (K / 2));
  dec.code8 = make_rsrc(code8 + f0 * (K / kBlock1), (N - f0) * (K / kBlock1));
  dec.c2s = make_rsrc(c2s, ((N * (K / kBlock1) + 255) / 256) * 4);
  dec.row_off = (uint32_t)(st * (K / 2));
  dec.blk = (uint32_t)(st * (K / kBlock1));
  dec.blk0 = (uint32_t)(f0 * (K / kBlock1));
  dec.mu = mu_p[0];
  dec.T = T;
  dec.t = st;

  FwdDec::Regs r0, r1;
  Acc acc;
  // adapter: Y += (s T) B^T, B [N, r] row-major -> element (f, j) at f*r + j
  gemm_prologue(dec, ring, nk, wrole, r0, r1, Bl, r, 1, N, Lm, M, r, f0, m0, st, wf, wmt, l32, h32, acc);
  gemm_main(dec, ring, nk, wrole, wf, wmt, l32, h32, r0, r1, acc);
  store_tile(Y, M, N, f0 + wf, m0 + wmt, l32, h32, acc);
}

__global__ __launch_bounds__(kThreads, 1) void k_gemm_dx(
    const uint32_t* __restrict__ codes, const uint8_t* __restrict__ code8,
    const float* __restrict__ c2s, const float* __restrict__ mu_p, int64_t N, int64_t K,
    const uint16_t* __restrict__ dY, int64_t M, const uint16_t* __restrict__ Lg,
    const uint16_t* __restrict__ Al, int32_t r, uint16_t* __restrict__ dX, Nf4Tables T) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h32 = lane >> 5;
  const int wf = (wave & 1) * 128, wmt = (wave >> 1) * 64;
  const bool wrole = tid < kStage;
  const int st = wrole ? tid : tid - kStage;
  int64_t tx, ty;
  tile_xy(tx, ty);
  const int64_t k0 = tx * BF, m0 = ty * BMT;  // output features = columns of W
  const uint32_t nk = (uint32_t)((N + BK - 1) / BK);

  ActRing ring;
  ring.init(dY, M, m0, N, wave, lane);
  DxDec dec;
  dec.codes = reinterpret_cast<const uint8_t*>(codes);
  dec.codes_bytes = N * (K / 2);
  dec.code8 = make_rsrc(code8, N * (K / kBlock1));
  dec.c2s = make_rsrc(c2s, ((N * (K / kBlock1) + 255) / 256) * 4);
  dec.row_bytes = (uint32_t)(K / 2);
  dec.nb_row = (uint32_t)(K / kBlock1);
  dec.N = (uint32_t)N;
  dec.mu = mu_p[0];
  load_unscaled_lut(T, dec.L);
  dec.t = st;
  {
    const int rg = st >> 5, kc = st & 31, e = kc & 7;
    const int64_t k = k0 + 8 * kc;
    dec.code_off = (k < K) ? (uint32_t)((8 * rg) * (K / 2) + k / 2) : kOOB;
    dec.own_row = (uint32_t)(8 * rg + e);
    dec.blk_off = (uint32_t)((8 * rg + e) * (K / kBlock1) + (k0 + 64 * (kc >> 3)) / kBlock1);
  }

  DxDec::Regs r0, r1;
  Acc acc;
  // adapter: dX += (s G) A, A [r, K] -> element (f = k, j) at j*K + k
  gemm_prologue(dec, ring, nk, wrole, r0, r1, Al, 1, K, K, Lg, M, r, k0, m0, st, wf, wmt, l32, h32, acc);
  gemm_main(dec, ring, nk, wrole, wf, wmt, l32, h32, r0, r1, acc);
  store_tile(dX, M, K, k0 + wf, m0 + wmt, l32, h32, acc);
}

}  // namespace

hipError_t launch_gemm_fwd(const uint32_t* codes, const uint8_t* code8, const float* c2s,
                           const float* mu, int64_t N, int64_t K, const uint16_t* X, int64_t M,
                           const uint16_t* L, const uint16_t* B, int32_t r, uint16_t* Y,
                           const Nf4Tables& T, hipStream_t st) {
  dim3 grid((unsigned)((N + BF - 1) / BF), (unsigned)((M + BMT - 1) / BMT));
  LaunchTimer t(4, st);
  hipExtLaunchKernelGGL(k_gemm_fwd, grid, dim3(kThreads), 0, st, t.start, t.stop, 0, codes, code8, c2s, mu, N, K, X, M,
                     L, B, r, Y, T);
  return hipGetLastError();
}

hipError_t launch_gemm_dx(const uint32_t* codes, const uint8_t* code8, const float* c2s,
                          const float* mu, int64_t N, int64_t K, const uint16_t* dY, int64_t M,
                          const uint16_t* Lg, const uint16_t* A, int32_t r, uint16_t* dX,
                          const Nf4Tables& T, hipStream_t st) {
  dim3 grid((unsigned)((K + BF - 1) / BF), (unsigned)((M + BMT - 1) / BMT));
  LaunchTimer t(5, st);
  hipExtLaunchKernelGGL(k_gemm_dx, grid, dim3(kThreads), 0, st, t.start, t.stop, 0, codes, code8, c2s, mu, N, K, dY, M,
                     Lg, A, r, dX, T);
  return hipGetLastError();
}

}  // namespace qlora
