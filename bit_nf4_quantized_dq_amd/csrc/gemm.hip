// Fused dequantize -> BF16 MFMA GEMMs for many tokens (M > 16).
//
// "QLoRA: Quantize Base Weights to 4-Bit", Section 3: the 4-bit weights stay in HBM; a
// tile is expanded to BF16 on chip and fed to the matrix units, and the adapter branch is
// added.  "QLoRA -- Fine-Tuning a 65B Model on One GPU", "Where the gradients actually go":
// the input gradient runs through the dequantized weights (dX = dY w_hat + s G A).
//
// Both kernels compute an output tile D[f][m] (f = output feature, m = token) with MFMA
// 16x16x32 BF16: the decoded weights are the A operand (rows f), activations the B operand
// (columns m), so each lane ends with 4 consecutive features of one token and stores 8 bytes.
//
//   forward : f = n (d_out), reduction over k (d_in).  W rows are k-contiguous, so a thread
//             decodes one (row, 64-block) = 8 code words with a per-block scaled BF16 table
//             (bit-exact w_hat) and writes 8 16-byte chunks of LDS row f.
//   dX      : f = k (d_in), reduction over n (d_out).  The quantization blocks now run along
//             the output dimension, so a thread decodes 8 rows x 8 columns with the unscaled
//             table, applies each row's constant in FP32, and writes the 8x8 tile transposed
//             (8 n-values per feature k) -- the transposed tile.
// Adapter term: after the main loop, ceil(r/32) extra reduction steps of width 32 multiply
// the prescaled BF16 side input (s T for forward, s G for dX) by B (forward) or A^T (dX).
//
// Tiling: 256 (features) x 256 (tokens) per workgroup, reduction step 64, 4 wavefronts in a
// 2 x 2 grid of 128 x 128 wavefront tiles (8 x 8 MFMA tiles, FP32 accumulators).  LDS holds
// two stages of a BF16 weight tile and a BF16 activation tile (4 x 32 KB); 16-byte chunks
// are XOR-swizzled by row so both the staging writes and the MFMA operand reads are free of
// bank conflicts.  Global loads are raw buffer loads (zero outside the tensor), so the
// steady-state loop has no branches; the last stage is peeled.
#include "qlora_device.h"
#include "qlora_host.h"

namespace qlora {
namespace {

constexpr int kThreads = 256;
constexpr int BF = 256;   // features per tile
constexpr int BMT = 256;  // tokens per tile
constexpr int BK = 64;    // reduction step
constexpr int kChunks = BK / 8;  // 16-byte chunks per LDS row

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kChunks + (chunk ^ ((row ^ (row >> 3)) & 7));
}

struct Smem {
  uint4 w[2][BF * kChunks];
  uint4 x[2][BMT * kChunks];
};

// ---- activation tile: rows = tokens (from m0), columns = reduction index (Kr in total)
struct ActRegs {
  uint4 v[8];
};

__device__ __forceinline__ void act_load(rsrc_t rp, int64_t Kr, int64_t k0, ActRegs& R) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = threadIdx.x + kThreads * i;
    const int row = c >> 3, ch = c & 7;
    const int64_t k = k0 + 8 * ch;
    const uint32_t off = (k < Kr) ? (uint32_t)((row * Kr + k) * 2) : kOOB;
    R.v[i] = bload16(rp, off);
  }
}

__device__ __forceinline__ void act_store(uint4* __restrict__ s, const ActRegs& R) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = threadIdx.x + kThreads * i;
    s[swz(c >> 3, c & 7)] = R.v[i];
  }
}

// ---- forward weight tile: thread t decodes row f0 + t, block kb (64 weights)
struct FwdRegs {
  uint4 c0, c1;
  uint32_t c8;
  float c2;
};

struct FwdSrc {
  rsrc_t codes;  // from row f0
  rsrc_t code8;  // whole tensor
  rsrc_t c2s;    // whole tensor
  int64_t row_bytes;  // K / 2
  int64_t nb_row;     // K / 64
  int64_t f0;
};

__device__ __forceinline__ void fwd_w_load(const FwdSrc& S, int64_t kb, FwdRegs& R) {
  const int t = threadIdx.x;
  const uint32_t off = (uint32_t)(t * S.row_bytes + kb * 32);
  R.c0 = bload16(S.codes, off);
  R.c1 = bload16(S.codes, off + 16);
  const int64_t blk = (S.f0 + t) * S.nb_row + kb;
  R.c8 = bload1(S.code8, (uint32_t)blk);
  R.c2 = __uint_as_float(bload4(S.c2s, (uint32_t)((blk >> 8) * 4)));
}

__device__ __forceinline__ void fwd_w_store(uint4* __restrict__ s, const FwdRegs& R, float mu,
                                            const Nf4Tables& T) {
  Lut L;
  build_scaled_lut(T, block_scale(R.c8, R.c2, mu), L);
  const uint32_t words[8] = {R.c0.x, R.c0.y, R.c0.z, R.c0.w, R.c1.x, R.c1.y, R.c1.z, R.c1.w};
  const int row = threadIdx.x;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    uint32_t o[4];
    decode8(words[c], L, o);
    s[swz(row, c)] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// ---- dX weight tile: thread t decodes rows n0 + 8*(t>>5) + i (i < 8), columns k0 + 8*(t&31) + e
struct DxRegs {
  uint32_t w[8];
  uint32_t c8[8];
  float c2[8];
};

struct DxSrc {
  rsrc_t codes;  // whole tensor
  rsrc_t code8;
  rsrc_t c2s;
  int64_t K;
  int64_t k0;
};

__device__ __forceinline__ void dx_w_load(const DxSrc& S, int64_t n0, DxRegs& R) {
  const int rg = threadIdx.x >> 5, kc = threadIdx.x & 31;
  const int64_t k = S.k0 + 8 * kc;
  const bool kok = k < S.K;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t n = n0 + 8 * rg + i;
    R.w[i] = bload4(S.codes, kok ? (uint32_t)((n * S.K + k) / 2) : kOOB);
    const int64_t blk = n * (S.K / kBlock1) + (k >> 6);
    R.c8[i] = bload1(S.code8, kok ? (uint32_t)blk : kOOB);
    R.c2[i] = __uint_as_float(bload4(S.c2s, kok ? (uint32_t)((blk >> 8) * 4) : kOOB));
  }
}

__device__ __forceinline__ void dx_w_store(uint4* __restrict__ s, const DxRegs& R, float mu, const Lut& L) {
  const int rg = threadIdx.x >> 5, kc = threadIdx.x & 31;
  float sc[8];
  uint32_t d[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    sc[i] = block_scale(R.c8[i], R.c2[i], mu);
    decode8(R.w[i], L, d[i]);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    uint32_t o[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t a = d[2 * p][e >> 1], b = d[2 * p + 1][e >> 1];
      const float fa = (e & 1) ? bf16hi_to_f32(a) : bf16lo_to_f32(a);
      const float fb = (e & 1) ? bf16hi_to_f32(b) : bf16lo_to_f32(b);
      o[p] = pack_bf16x2(fa * sc[2 * p], fb * sc[2 * p + 1]);
    }
    s[swz(8 * kc + e, rg)] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// ---- MFMA on one LDS stage: two 32-wide reduction halves, 8 x 8 tiles per wavefront
__device__ __forceinline__ void mma_stage(const uint4* __restrict__ sw, const uint4* __restrict__ sx,
                                          int wf, int wmt, int lr, int lg, f32x4_t (&acc)[8][8]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    bf16x8_t a[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = as_bf16x8(sw[swz(wf + 16 * i + lr, 4 * h + lg)]);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bf16x8_t b = as_bf16x8(sx[swz(wmt + 16 * j + lr, 4 * h + lg)]);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i][j] = mfma16x16x32(a[i], b, acc[i][j]);
    }
  }
}

// Gather 8 BF16 values p[0], p[stride], ... (predicated) into one MFMA operand.
__device__ __forceinline__ bf16x8_t gather8(const uint16_t* __restrict__ p, int64_t stride, int valid) {
  uint32_t v[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t lo = (2 * q < valid) ? p[(2 * q) * stride] : 0u;
    const uint32_t hi = (2 * q + 1 < valid) ? p[(2 * q + 1) * stride] : 0u;
    v[q] = lo | (hi << 16);
  }
  return as_bf16x8(v);
}

// Adapter K-slices: acc[f][m] += sum_j Wl[f][j] * Lm[m][j], j < r.  Wl element (f, j) is at
// wl[f * wl_fs + j * wl_js]; Lm is [M, r] row-major.
__device__ __forceinline__ void lora_slices(const uint16_t* __restrict__ wl, int64_t wl_fs, int64_t wl_js,
                                            int64_t F, const uint16_t* __restrict__ Lm, int64_t M,
                                            int32_t r, int64_t f0, int64_t m0, int lr, int lg,
                                            f32x4_t (&acc)[8][8]) {
  for (int32_t j0 = 0; j0 < r; j0 += 32) {
    const int32_t jj = j0 + 8 * lg;
    const int valid = (r - jj) > 8 ? 8 : (r - jj > 0 ? r - jj : 0);
    bf16x8_t a[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t f = f0 + 16 * i + lr;
      a[i] = gather8(wl + (f < F ? f : 0) * wl_fs + (int64_t)jj * wl_js, wl_js, f < F ? valid : 0);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t m = m0 + 16 * j + lr;
      const bf16x8_t b = gather8(Lm + (m < M ? m : 0) * r + jj, 1, m < M ? valid : 0);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i][j] = mfma16x16x32(a[i], b, acc[i][j]);
    }
  }
}

// Store D[f][m] tile: lane holds features f = f0 + 16 i + 4 lg + v (v < 4) of token m.
__device__ __forceinline__ void store_tile(uint16_t* __restrict__ Y, int64_t M, int64_t F, int64_t f0,
                                           int64_t m0, int lr, int lg, const f32x4_t (&acc)[8][8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t m = m0 + 16 * j + lr;
    if (m >= M) continue;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t f = f0 + 16 * i + 4 * lg;
      if (f < F) {
        const uint32_t lo = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
        const uint32_t hi = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
        *reinterpret_cast<uint2*>(Y + m * F + f) = make_uint2(lo, hi);
      }
    }
  }
}

__global__ __launch_bounds__(kThreads, 1) void k_gemm_fwd(
    const uint32_t* __restrict__ codes, const uint8_t* __restrict__ code8,
    const float* __restrict__ c2s, const float* __restrict__ mu_p, int64_t N, int64_t K,
    const uint16_t* __restrict__ X, int64_t M, const uint16_t* __restrict__ Lm,
    const uint16_t* __restrict__ Bl, int32_t r, uint16_t* __restrict__ Y, Nf4Tables T) {
  extern __shared__ uint4 smem_raw[];
  Smem& S = *reinterpret_cast<Smem*>(smem_raw);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int wf = (wave >> 1) * 128, wmt = (wave & 1) * 128;
  const int64_t f0 = (int64_t)blockIdx.x * BF;
  const int64_t m0 = (int64_t)blockIdx.y * BMT;
  const float mu = mu_p[0];
  const int64_t nkb = K / BK;

  const rsrc_t xr = make_rsrc(X + m0 * K, (M - m0) * K * 2);
  FwdSrc ws;
  ws.codes = make_rsrc(reinterpret_cast<const uint8_t*>(codes) + f0 * (K / 2), (N - f0) * (K / 2));
  ws.code8 = make_rsrc(code8, N * (K / kBlock1));
  ws.c2s = make_rsrc(c2s, ((N * (K / kBlock1) + 255) / 256) * 4);
  ws.row_bytes = K / 2;
  ws.nb_row = K / kBlock1;
  ws.f0 = f0;

  f32x4_t acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  ActRegs ar;
  FwdRegs wr;
  act_load(xr, K, 0, ar);
  fwd_w_load(ws, 0, wr);
  act_store(S.x[0], ar);
  fwd_w_store(S.w[0], wr, mu, T);
  __syncthreads();

  for (int64_t kb = 0; kb + 1 < nkb; ++kb) {
    const int buf = kb & 1;
    act_load(xr, K, (kb + 1) * BK, ar);
    fwd_w_load(ws, kb + 1, wr);
    mma_stage(S.w[buf], S.x[buf], wf, wmt, lr, lg, acc);
    act_store(S.x[buf ^ 1], ar);
    fwd_w_store(S.w[buf ^ 1], wr, mu, T);
    __syncthreads();
  }
  mma_stage(S.w[(nkb - 1) & 1], S.x[(nkb - 1) & 1], wf, wmt, lr, lg, acc);
  // adapter: Y += (s T) B^T, B [N, r] row-major -> element (f, j) at f*r + j
  lora_slices(Bl, r, 1, N, Lm, M, r, f0 + wf, m0 + wmt, lr, lg, acc);
  store_tile(Y, M, N, f0 + wf, m0 + wmt, lr, lg, acc);
}

__global__ __launch_bounds__(kThreads, 1) void k_gemm_dx(
    const uint32_t* __restrict__ codes, const uint8_t* __restrict__ code8,
    const float* __restrict__ c2s, const float* __restrict__ mu_p, int64_t N, int64_t K,
    const uint16_t* __restrict__ dY, int64_t M, const uint16_t* __restrict__ Lg,
    const uint16_t* __restrict__ Al, int32_t r, uint16_t* __restrict__ dX, Nf4Tables T) {
  extern __shared__ uint4 smem_raw[];
  Smem& S = *reinterpret_cast<Smem*>(smem_raw);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int wf = (wave >> 1) * 128, wmt = (wave & 1) * 128;
  const int64_t k0 = (int64_t)blockIdx.x * BF;  // output features = columns of W
  const int64_t m0 = (int64_t)blockIdx.y * BMT;
  const float mu = mu_p[0];
  const int64_t nnb = (N + BK - 1) / BK;
  Lut L;
  load_unscaled_lut(T, L);

  const rsrc_t yr = make_rsrc(dY + m0 * N, (M - m0) * N * 2);
  DxSrc ws;
  ws.codes = make_rsrc(codes, N * (K / 2));
  ws.code8 = make_rsrc(code8, N * (K / kBlock1));
  ws.c2s = make_rsrc(c2s, ((N * (K / kBlock1) + 255) / 256) * 4);
  ws.K = K;
  ws.k0 = k0;

  f32x4_t acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  ActRegs ar;
  DxRegs wr;
  act_load(yr, N, 0, ar);
  dx_w_load(ws, 0, wr);
  act_store(S.x[0], ar);
  dx_w_store(S.w[0], wr, mu, L);
  __syncthreads();

  for (int64_t nb = 0; nb + 1 < nnb; ++nb) {
    const int buf = nb & 1;
    act_load(yr, N, (nb + 1) * BK, ar);
    dx_w_load(ws, (nb + 1) * BK, wr);
    mma_stage(S.w[buf], S.x[buf], wf, wmt, lr, lg, acc);
    act_store(S.x[buf ^ 1], ar);
    dx_w_store(S.w[buf ^ 1], wr, mu, L);
    __syncthreads();
  }
  mma_stage(S.w[(nnb - 1) & 1], S.x[(nnb - 1) & 1], wf, wmt, lr, lg, acc);
  // adapter: dX += (s G) A, A [r, K] -> element (f = k, j) at j*K + k
  lora_slices(Al, 1, K, K, Lg, M, r, k0 + wf, m0 + wmt, lr, lg, acc);
  store_tile(dX, M, K, k0 + wf, m0 + wmt, lr, lg, acc);
}

constexpr size_t kSmemBytes = sizeof(Smem);

hipError_t set_smem(const void* fn, bool& done) {
  if (done) return hipSuccess;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kSmemBytes);
  if (e == hipSuccess) done = true;
  return e;
}

}  // namespace

hipError_t launch_gemm_fwd(const uint32_t* codes, const uint8_t* code8, const float* c2s,
                           const float* mu, int64_t N, int64_t K, const uint16_t* X, int64_t M,
                           const uint16_t* L, const uint16_t* B, int32_t r, uint16_t* Y,
                           const Nf4Tables& T, hipStream_t st) {
  static bool done = false;
  hipError_t e = set_smem(reinterpret_cast<const void*>(&k_gemm_fwd), done);
  if (e != hipSuccess) return e;
  dim3 grid((unsigned)((N + BF - 1) / BF), (unsigned)((M + BMT - 1) / BMT));
  LaunchTimer t(4, st);
  hipLaunchKernelGGL(k_gemm_fwd, grid, dim3(kThreads), kSmemBytes, st, codes, code8, c2s, mu, N, K,
                     X, M, L, B, r, Y, T);
  return hipGetLastError();
}

hipError_t launch_gemm_dx(const uint32_t* codes, const uint8_t* code8, const float* c2s,
                          const float* mu, int64_t N, int64_t K, const uint16_t* dY, int64_t M,
                          const uint16_t* Lg, const uint16_t* A, int32_t r, uint16_t* dX,
                          const Nf4Tables& T, hipStream_t st) {
  static bool done = false;
  hipError_t e = set_smem(reinterpret_cast<const void*>(&k_gemm_dx), done);
  if (e != hipSuccess) return e;
  dim3 grid((unsigned)((K + BF - 1) / BF), (unsigned)((M + BMT - 1) / BMT));
  LaunchTimer t(5, st);
  hipLaunchKernelGGL(k_gemm_dx, grid, dim3(kThreads), kSmemBytes, st, codes, code8, c2s, mu, N, K,
                     dY, M, Lg, A, r, dX, T);
  return hipGetLastError();
}

}  // namespace qlora
