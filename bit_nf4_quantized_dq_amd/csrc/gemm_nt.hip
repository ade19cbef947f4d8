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
// step 32.  Both operand tiles stream through four-slot LDS rings filled by direct
// buffer->LDS loads issued three steps ahead; each step is: read the first half of the
// step's operands, issue the loads of step kb+3, run the deferred second-half MFMAs of step
// kb-1, read the second half, run the first-half MFMAs, wait for this wavefront's loads of
// step kb+1, one barrier.  The step loop is
// unrolled four times so that each ring slot is a distinct LDS array known at compile time,
// which lets the compiler wait only for the slot an access touches.  Rows are 4 chunks of
// 16 bytes, XOR-swizzled by (row >> 2) & 3: the LDS serves 16 lanes x 16 bytes per clock
// from 64 banks, and the 16 rows x one chunk of an MFMA operand read then cover all 256
// bytes exactly once; the ring writes (1 KB contiguous per load) are conflict-free anyway.  Out-of-range rows or
// reduction columns read as zero (raw buffer loads), so no tail needs a branch in the loop.
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

// Two rings of four 16 KB slots (128 KB).
__shared__ uint4 s_a0[kSlot], s_a1[kSlot], s_a2[kSlot], s_a3[kSlot];
__shared__ uint4 s_b0[kSlot], s_b1[kSlot], s_b2[kSlot], s_b3[kSlot];

template <int I> __device__ __forceinline__ uint4* abuf() {
  return I == 0 ? s_a0 : (I == 1 ? s_a1 : (I == 2 ? s_a2 : s_a3));
}
template <int I> __device__ __forceinline__ uint4* bbuf() {
  return I == 0 ? s_b0 : (I == 1 ? s_b1 : (I == 2 ? s_b2 : s_b3));
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
  uint32_t base[2];  // byte offset of the lane's chunk at reduction index 0; kOOB past the rows
  uint32_t col[2];   // the lane's first reduction index within a step
  uint32_t Kr;
  int wave;

  __device__ __forceinline__ void init(const uint16_t* P, int64_t rows_total, int64_t row0, int64_t Kr_, int w,
                                       int lane) {
    const int64_t rows = rows_total - row0 < 256 ? rows_total - row0 : 256;
    r = make_rsrc(P + row0 * Kr_, rows * Kr_ * 2);
    Kr = (uint32_t)Kr_;
    wave = w;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int row = 16 * (2 * w + j) + (lane >> 2);
      const int lc = (lane & 3) ^ ((row >> 2) & 3);
      col[j] = 8 * lc;
      base[j] = row < rows ? (uint32_t)(row * Kr_ * 2 + 16 * lc) : kOOB;
    }
  }
  __device__ __forceinline__ void issue(uint4* slot, uint32_t kb) const {
    const uint32_t k0 = kb * BK;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t off = (base[j] != kOOB && k0 + col[j] < Kr) ? base[j] + 2 * k0 : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(slot + (2 * wave + j) * 64), 16, off, 0, 0, 0);
    }
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
__device__ __forceinline__ void mma_step(const uint4* __restrict__ sa, const uint4* __restrict__ sb, int wf,
                                         int wmt, int l32, int h32, Acc& acc) {
  Ops o0, o1;
  read_ops(sa, sb, 0, wf, wmt, l32, h32, o0);
  read_ops(sa, sb, 1, wf, wmt, l32, h32, o1);
  mma(o0, acc);
  mma(o1, acc);
}

// Adapter slices of 32: acc[f][m] += sum_j Wl(f, j) * L[m][j], Wl(f, j) at f*wl_fs + j*wl_js
// (elements), L [M, r] row-major; element loads (any r, any stride), staged through slot 3.
// Threads 0-255 load feature row f0 + t, threads 256-511 token row m0 + t - 256.
__device__ __forceinline__ void adapter(const uint16_t* __restrict__ wl, int64_t wl_fs, int64_t wl_js, int64_t F,
                                        const uint16_t* __restrict__ Lm, int64_t M, int32_t r, int64_t f0, int64_t m0,
                                        int tid, int wf, int wmt, int l32, int h32, Acc& acc) {
  const bool wside = tid < 256;
  const int row = wside ? tid : tid - 256;
  const rsrc_t rw = make_rsrc(wl, (F - 1) * wl_fs * 2 + (int64_t)r * wl_js * 2);
  const rsrc_t rm = make_rsrc(Lm, M * (int64_t)r * 2);
  for (int32_t j0 = 0; j0 < r; j0 += BK) {
    uint32_t e[BK];
    if (wside) {
      const int64_t f = f0 + row;
#pragma unroll
      for (int q = 0; q < BK; ++q) {
        const bool ok = f < F && j0 + q < r;
        e[q] = __builtin_amdgcn_raw_buffer_load_b16(rw, ok ? (int)((f * wl_fs + (int64_t)(j0 + q) * wl_js) * 2) : (int)kOOB, 0, 0);
      }
    } else {
      const int64_t m = m0 + row;
#pragma unroll
      for (int q = 0; q < BK; ++q) {
        const bool ok = m < M && j0 + q < r;
        e[q] = __builtin_amdgcn_raw_buffer_load_b16(rm, ok ? (int)((m * r + j0 + q) * 2) : (int)kOOB, 0, 0);
      }
    }
    uint4* dst = wside ? abuf<3>() : bbuf<3>();
    if (j0 > 0) lds_barrier();  // the previous slice's MFMA reads are done
#pragma unroll
    for (int c = 0; c < kChunks; ++c)
      dst[swz(row, c)] = make_uint4((e[8 * c + 0] & 0xFFFFu) | (e[8 * c + 1] << 16), (e[8 * c + 2] & 0xFFFFu) | (e[8 * c + 3] << 16),
                                    (e[8 * c + 4] & 0xFFFFu) | (e[8 * c + 5] << 16), (e[8 * c + 6] & 0xFFFFu) | (e[8 * c + 7] << 16));
    lds_barrier();
    mma_step(abuf<3>(), bbuf<3>(), wf, wmt, l32, h32, acc);
  }
}

// Store C (32x32 layout): register 4q + v of tile (i, j) holds feature
// f = f0 + 32 i + 8 q + 4 h32 + v of token m = m0 + 32 j + l32; output is [M, F] BF16.
__device__ __forceinline__ void store_tile(uint16_t* __restrict__ Y, int64_t M, int64_t F, int64_t f0, int64_t m0,
                                           int l32, int h32, const Acc& acc) {
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

// Consecutive workgroups are dealt round-robin to the 8 XCDs (each with its own L2):
// renumber so that one XCD gets a contiguous run of tiles in feature-fastest order.
__device__ __forceinline__ void tile_xy(int64_t& tx, int64_t& ty) {
  const uint32_t gx = gridDim.x, n = gridDim.x * gridDim.y;
  uint32_t L = blockIdx.x + gx * blockIdx.y;
  if ((n & 7) == 0) L = (L & 7) * (n >> 3) + (L >> 3);
  tx = L % gx;
  ty = L / gx;
}

// Ring step kb (slot S), entered right after the barrier that published it.  The second
// half (ks = 1) of the previous step's MFMAs was deferred: its operands are in `o1`, so
// those MFMAs run while this step's operand reads are in flight, and the wavefronts never
// sit on an LDS read directly after a barrier.
template <int S>
__device__ __forceinline__ void nt_step(const Ring& ra, const Ring& rb, uint32_t kb, uint32_t nk, int wf, int wmt,
                                        int l32, int h32, Ops& o1, Acc& acc) {
  Ops o0;
  read_ops(abuf<S>(), bbuf<S>(), 0, wf, wmt, l32, h32, o0);
  if (kb + 3 < nk) {
    ra.issue(abuf<(S + 3) % 4>(), kb + 3);
    rb.issue(bbuf<(S + 3) % 4>(), kb + 3);
  }
  mma(o1, acc);  // ks = 1 of step kb - 1
  read_ops(abuf<S>(), bbuf<S>(), 1, wf, wmt, l32, h32, o1);
  mma(o0, acc);
  // this wavefront's loads of step kb+1 are complete (steps kb+2, kb+3 may be pending)
  if (kb + 3 < nk) wait_vm<8>();
  else if (kb + 2 < nk) wait_vm<4>();
  else wait_vm<0>();
  lds_barrier();
}

__global__ __launch_bounds__(kThreads, 1) void k_gemm_nt(const uint16_t* __restrict__ A, int64_t F,
                                                         const uint16_t* __restrict__ B, int64_t M, int64_t Kr,
                                                         const uint16_t* __restrict__ wl, int64_t wl_fs,
                                                         int64_t wl_js, const uint16_t* __restrict__ Lm, int32_t r,
                                                         uint16_t* __restrict__ C) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h32 = lane >> 5;
  const int wf = (wave & 1) * 128, wmt = (wave >> 1) * 64;
  int64_t tx, ty;
  tile_xy(tx, ty);
  const int64_t f0 = tx * BF, m0 = ty * BMT;
  const uint32_t nk = (uint32_t)((Kr + BK - 1) / BK);

  Ring ra, rb;
  ra.init(A, F, f0, Kr, wave, lane);
  rb.init(B, M, m0, Kr, wave, lane);
  // steps 0..2 in flight while the adapter slices run through slot 3
  ra.issue(abuf<0>(), 0);
  rb.issue(bbuf<0>(), 0);
  if (nk > 1) {
    ra.issue(abuf<1>(), 1);
    rb.issue(bbuf<1>(), 1);
  }
  if (nk > 2) {
    ra.issue(abuf<2>(), 2);
    rb.issue(bbuf<2>(), 2);
  }
  Acc acc;
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = f32x16_t{};
  adapter(wl, wl_fs, wl_js, F, Lm, M, r, f0, m0, tid, wf, wmt, l32, h32, acc);
  wait_vm<0>();
  lds_barrier();  // step 0 landed everywhere; the adapter's reads of slot 3 are done

  Ops o1;  // deferred second half of the previous step: none before step 0
#pragma unroll
  for (int i = 0; i < TI; ++i) o1.a[i] = bf16x8_t{};
#pragma unroll
  for (int j = 0; j < TJ; ++j) o1.b[j] = bf16x8_t{};
  for (uint32_t kb = 0; kb < nk; kb += 4) {
    nt_step<0>(ra, rb, kb + 0, nk, wf, wmt, l32, h32, o1, acc);
    if (kb + 1 >= nk) break;
    nt_step<1>(ra, rb, kb + 1, nk, wf, wmt, l32, h32, o1, acc);
    if (kb + 2 >= nk) break;
    nt_step<2>(ra, rb, kb + 2, nk, wf, wmt, l32, h32, o1, acc);
    if (kb + 3 >= nk) break;
    nt_step<3>(ra, rb, kb + 3, nk, wf, wmt, l32, h32, o1, acc);
  }
  mma(o1, acc);  // ks = 1 of the last step
  store_tile(C, M, F, f0 + wf, m0 + wmt, l32, h32, acc);
}

}  // namespace

hipError_t launch_gemm_nt(const uint16_t* A, int64_t F, const uint16_t* B, int64_t M, int64_t Kr,
                          const uint16_t* wl, int64_t wl_fs, int64_t wl_js, const uint16_t* L, int32_t r,
                          uint16_t* C, int kernel_id, hipStream_t st) {
  dim3 grid((unsigned)((F + BF - 1) / BF), (unsigned)((M + BMT - 1) / BMT));
  LaunchTimer t(kernel_id, st);
  hipExtLaunchKernelGGL(k_gemm_nt, grid, dim3(kThreads), 0, st, t.start, t.stop, 0, A, F, B, M, Kr, wl, wl_fs, wl_js, L, r, C);
  return hipGetLastError();
}

}  // namespace qlora
