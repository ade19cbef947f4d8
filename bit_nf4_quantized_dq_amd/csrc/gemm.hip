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
// Adapter term: ceil(r/32) extra reduction steps of width 32 multiply the prescaled BF16
// side input (s T for forward, s G for dX) by B (forward) or A^T (dX); they run first,
// through the second LDS stage buffer, so the accumulators start from the adapter term.
//
// Tiling: 256 (features) x 256 (tokens) per workgroup, reduction step 64, 8 wavefronts
// (two per SIMD) in a 2 x 4 grid of 128 x 64 wavefront tiles (8 x 4 MFMA tiles, 128 FP32
// accumulators per lane).  Wavefronts 0-3 stage (decode) the weight tile, 4-7 stage the
// activation tile, through one shared prefetch register buffer; every wavefront then runs
// its share of the MFMAs, so the decode VALU work of one wavefront overlaps the matrix work
// of the other wavefront on its SIMD.  LDS holds two stages of both tiles (4 x 32 KB);
// 16-byte chunks are XOR-swizzled by row so the staging writes and the operand reads are
// free of bank conflicts.  Global loads are raw buffer loads (zero outside the tensor), so
// the steady-state loop has no data-dependent branches; the last stage is peeled.
#include "qlora_device.h"
#include "qlora_host.h"

namespace qlora {
namespace {

constexpr int kThreads = 512;
constexpr int kStage = 256;      // threads of each staging role
constexpr int BF = 256;          // features per tile
constexpr int BMT = 256;         // tokens per tile
constexpr int BK = 64;           // reduction step
constexpr int kChunks = BK / 8;  // 16-byte chunks per LDS row
constexpr int TI = 8, TJ = 4;    // 16x16 MFMA tiles per wavefront: 128 features x 64 tokens
typedef f32x4_t Acc[TI][TJ];

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kChunks + (chunk ^ ((row ^ (row >> 3)) & 7));
}

struct Smem {
  uint4 w[2][BF * kChunks];
  uint4 x[2][BMT * kChunks];
};

// One staging thread's global loads between issue and the LDS write (either role).
struct Pre {
  uint4 v[8];
};

// ---- activation tile: rows = tokens (from m0), columns = reduction index (Kr in total)
__device__ __forceinline__ void act_load(rsrc_t rp, uint32_t Kr, uint32_t k0, int t, Pre& R) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = t + kStage * i;
    const uint32_t row = c >> 3, k = k0 + 8 * (c & 7);
    R.v[i] = bload16(rp, (k < Kr) ? (row * Kr + k) * 2 : kOOB);
  }
}

__device__ __forceinline__ void act_store(uint4* __restrict__ s, int t, const Pre& R) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = t + kStage * i;
    s[swz(c >> 3, c & 7)] = R.v[i];
  }
}

// ---- forward weight tile: thread t decodes row f0 + t, block kb (64 weights)
struct FwdSrc {
  rsrc_t codes;  // from row f0
  rsrc_t code8;  // from block f0 * nb_row
  rsrc_t c2s;    // whole tensor
  uint32_t row_bytes;  // K / 2
  uint32_t nb_row;     // K / 64
  uint32_t blk0;       // f0 * nb_row
};

__device__ __forceinline__ void fwd_w_load(const FwdSrc& S, uint32_t kb, int t, Pre& R) {
  const uint32_t off = t * S.row_bytes + kb * 32;
  R.v[0] = bload16(S.codes, off);
  R.v[1] = bload16(S.codes, off + 16);
  const uint32_t lb = t * S.nb_row + kb;
  R.v[2].x = bload1(S.code8, lb);
  R.v[2].y = bload4(S.c2s, ((S.blk0 + lb) >> 8) * 4);
}

__device__ __forceinline__ void fwd_w_store(uint4* __restrict__ s, int t, const Pre& R, float mu,
                                            const Nf4Tables& T) {
  Lut L;
  build_scaled_lut(T, block_scale(R.v[2].x, __uint_as_float(R.v[2].y), mu), L);
  const uint32_t words[8] = {R.v[0].x, R.v[0].y, R.v[0].z, R.v[0].w, R.v[1].x, R.v[1].y, R.v[1].z, R.v[1].w};
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    uint32_t o[4];
    decode8(words[c], L, o);
    s[swz(t, c)] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// ---- dX weight tile: thread t decodes rows n0 + 8*(t>>5) + i (i < 8), columns k0 + 8*(t&31) + e
struct DxSrc {
  rsrc_t codes;  // whole tensor
  rsrc_t code8;
  rsrc_t c2s;
  uint32_t row_bytes;  // K / 2
  uint32_t nb_row;     // K / 64
  uint32_t code_off;   // this thread's offset of row 8*rg, column k0 + 8*kc (kOOB when past K)
  uint32_t blk_off;    // this thread's block index of row 8*rg
};

__device__ __forceinline__ void dx_w_load(const DxSrc& S, uint32_t n0, Pre& R) {
  uint32_t* w = reinterpret_cast<uint32_t*>(&R.v[0]);   // 8 code words
  uint32_t* c8 = reinterpret_cast<uint32_t*>(&R.v[2]);  // 8 code8
  uint32_t* c2 = reinterpret_cast<uint32_t*>(&R.v[4]);  // 8 c2s bits
  const bool kok = S.code_off != kOOB;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t n = n0 + i;
    w[i] = bload4(S.codes, kok ? S.code_off + n * S.row_bytes : kOOB);
    const uint32_t blk = S.blk_off + n * S.nb_row;
    c8[i] = bload1(S.code8, kok ? blk : kOOB);
    c2[i] = bload4(S.c2s, kok ? (blk >> 8) * 4 : kOOB);
  }
}

__device__ __forceinline__ void dx_w_store(uint4* __restrict__ s, int t, const Pre& R, float mu, const Lut& L) {
  const int rg = t >> 5, kc = t & 31;
  const uint32_t* w = reinterpret_cast<const uint32_t*>(&R.v[0]);
  const uint32_t* c8 = reinterpret_cast<const uint32_t*>(&R.v[2]);
  const uint32_t* c2 = reinterpret_cast<const uint32_t*>(&R.v[4]);
  uint32_t o[8][4];  // o[e][p]: BF16 pair (rows 2p, 2p+1) of column e
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float sa = block_scale(c8[2 * p], __uint_as_float(c2[2 * p]), mu);
    const float sb = block_scale(c8[2 * p + 1], __uint_as_float(c2[2 * p + 1]), mu);
    uint32_t da[4], db[4];
    decode8(w[2 * p], L, da);
    decode8(w[2 * p + 1], L, db);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t a = da[e >> 1], b = db[e >> 1];
      const float fa = (e & 1) ? bf16hi_to_f32(a) : bf16lo_to_f32(a);
      const float fb = (e & 1) ? bf16hi_to_f32(b) : bf16lo_to_f32(b);
      o[e][p] = pack_bf16x2(fa * sa, fb * sb);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) s[swz(8 * kc + e, rg)] = make_uint4(o[e][0], o[e][1], o[e][2], o[e][3]);
}

// ---- MFMA on one LDS stage: two 32-wide reduction halves
__device__ __forceinline__ void mma_stage(const uint4* __restrict__ sw, const uint4* __restrict__ sx,
                                          int wf, int wmt, int lr, int lg, Acc& acc) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    __builtin_amdgcn_sched_barrier(0);
    bf16x8_t a[TI], b[TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i) a[i] = as_bf16x8(sw[swz(wf + 16 * i + lr, 4 * h + lg)]);
#pragma unroll
    for (int j = 0; j < TJ; ++j) b[j] = as_bf16x8(sx[swz(wmt + 16 * j + lr, 4 * h + lg)]);
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) acc[i][j] = mfma16x16x32(a[i], b[j], acc[i][j]);
  }
}

// Adapter K-slices: acc[f][m] += sum_j Wl[f][j] * Lm[m][j], j < r, in slices of 32 j.
// Each slice is staged through an LDS stage buffer (weights side by wavefronts 0-3, token
// side by 4-7; one row of 32 values per thread, element loads with out-of-range zeros) and
// multiplied like one 32-wide half of a main-loop stage.  Wl element (f, j) is at
// f * wl_fs + j * wl_js (elements); Lm is [M, r] row-major.
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
    bf16x8_t a[TI], b[TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i) a[i] = as_bf16x8(sw[swz(wf + 16 * i + lr, lg)]);
#pragma unroll
    for (int j = 0; j < TJ; ++j) b[j] = as_bf16x8(sx[swz(wmt + 16 * j + lr, lg)]);
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) acc[i][j] = mfma16x16x32(a[i], b[j], acc[i][j]);
  }
}

// Store D[f][m] tile: lane holds features f = f0 + 16 i + 4 lg + v (v < 4) of token m.
__device__ __forceinline__ void store_tile(uint16_t* __restrict__ Y, int64_t M, int64_t F, int64_t f0,
                                           int64_t m0, int lr, int lg, const Acc& acc) {
#pragma unroll
  for (int j = 0; j < TJ; ++j) {
    const int64_t m = m0 + 16 * j + lr;
    if (m >= M) continue;
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const int64_t f = f0 + 16 * i + 4 * lg;
      if (f < F) {
        const uint32_t lo = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
        const uint32_t hi = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
        *reinterpret_cast<uint2*>(Y + m * F + f) = make_uint2(lo, hi);
      }
    }
  }
}

__device__ __forceinline__ void zero_acc(Acc& acc) {
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
}

__global__ __launch_bounds__(kThreads, 1) void k_gemm_fwd(
    const uint32_t* __restrict__ codes, const uint8_t* __restrict__ code8,
    const float* __restrict__ c2s, const float* __restrict__ mu_p, int64_t N, int64_t K,
    const uint16_t* __restrict__ X, int64_t M, const uint16_t* __restrict__ Lm,
    const uint16_t* __restrict__ Bl, int32_t r, uint16_t* __restrict__ Y, Nf4Tables T) {
  extern __shared__ uint4 smem_raw[];
  Smem& S = *reinterpret_cast<Smem*>(smem_raw);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int wf = (wave & 1) * 128, wmt = (wave >> 1) * 64;
  const bool wrole = tid < kStage;  // wavefronts 0-3 stage weights, 4-7 activations
  const int st = wrole ? tid : tid - kStage;
  const int64_t f0 = (int64_t)blockIdx.x * BF;
  const int64_t m0 = (int64_t)blockIdx.y * BMT;
  const float mu = mu_p[0];
  const uint32_t nkb = (uint32_t)(K / BK);

  const rsrc_t xr = make_rsrc(X + m0 * K, (M - m0) * K * 2);
  FwdSrc ws;
  ws.codes = make_rsrc(reinterpret_cast<const uint8_t*>(codes) + f0 * (K / 2), (N - f0) * (K / 2));
  ws.code8 = make_rsrc(code8 + f0 * (K / kBlock1), (N - f0) * (K / kBlock1));
  ws.c2s = make_rsrc(c2s, ((N * (K / kBlock1) + 255) / 256) * 4);
  ws.row_bytes = (uint32_t)(K / 2);
  ws.nb_row = (uint32_t)(K / kBlock1);
  ws.blk0 = (uint32_t)(f0 * (K / kBlock1));

  Pre pre;
  if (wrole) fwd_w_load(ws, 0, st, pre);
  else act_load(xr, (uint32_t)K, 0, st, pre);

  Acc acc;
  zero_acc(acc);
  // adapter: Y += (s T) B^T, B [N, r] row-major -> element (f, j) at f*r + j
  lora_slices(Bl, r, 1, N, Lm, M, r, f0, m0, wrole, st, S.w[1], S.x[1], wf, wmt, lr, lg, acc);

  if (wrole) fwd_w_store(S.w[0], st, pre, mu, T);
  else act_store(S.x[0], st, pre);
  __syncthreads();

  for (uint32_t kb = 0; kb + 1 < nkb; ++kb) {
    const int buf = kb & 1;
    if (wrole) fwd_w_load(ws, kb + 1, st, pre);
    else act_load(xr, (uint32_t)K, (kb + 1) * BK, st, pre);
    mma_stage(S.w[buf], S.x[buf], wf, wmt, lr, lg, acc);
    if (wrole) fwd_w_store(S.w[buf ^ 1], st, pre, mu, T);
    else act_store(S.x[buf ^ 1], st, pre);
    __syncthreads();
  }
  mma_stage(S.w[(nkb - 1) & 1], S.x[(nkb - 1) & 1], wf, wmt, lr, lg, acc);
  store_tile(Y, M, N, f0 + wf, m0 + wmt, lr, lg, acc);
}

__global__ __launch_bounds__(kThreads, 1) void k_gemm_dx(
    const uint32_t* __restrict__ codes, const uint8_t* __restrict__ code8,
    const float* __restrict__ c2s, const float* __restrict__ mu_p, int64_t N, int64_t K,
    const uint16_t* __restrict__ dY, int64_t M, const uint16_t* __restrict__ Lg,
    const uint16_t* __restrict__ Al, int32_t r, uint16_t* __restrict__ dX, Nf4Tables T) {
  extern __shared__ uint4 smem_raw[];
  Smem& S = *reinterpret_cast<Smem*>(smem_raw);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int wf = (wave & 1) * 128, wmt = (wave >> 1) * 64;
  const bool wrole = tid < kStage;
  const int st = wrole ? tid : tid - kStage;
  const int64_t k0 = (int64_t)blockIdx.x * BF;  // output features = columns of W
  const int64_t m0 = (int64_t)blockIdx.y * BMT;
  const float mu = mu_p[0];
  const uint32_t nnb = (uint32_t)((N + BK - 1) / BK);
  Lut L;
  load_unscaled_lut(T, L);

  const rsrc_t yr = make_rsrc(dY + m0 * N, (M - m0) * N * 2);
  DxSrc ws;
  ws.codes = make_rsrc(codes, N * (K / 2));
  ws.code8 = make_rsrc(code8, N * (K / kBlock1));
  ws.c2s = make_rsrc(c2s, ((N * (K / kBlock1) + 255) / 256) * 4);
  ws.row_bytes = (uint32_t)(K / 2);
  ws.nb_row = (uint32_t)(K / kBlock1);
  {
    const int rg = st >> 5, kc = st & 31;
    const int64_t k = k0 + 8 * kc;
    ws.code_off = (k < K) ? (uint32_t)((8 * rg) * (K / 2) + k / 2) : kOOB;
    ws.blk_off = (uint32_t)((8 * rg) * (K / kBlock1) + k / kBlock1);
  }

  Pre pre;
  if (wrole) dx_w_load(ws, 0, pre);
  else act_load(yr, (uint32_t)N, 0, st, pre);

  Acc acc;
  zero_acc(acc);
  // adapter: dX += (s G) A, A [r, K] -> element (f = k, j) at j*K + k
  lora_slices(Al, 1, K, K, Lg, M, r, k0, m0, wrole, st, S.w[1], S.x[1], wf, wmt, lr, lg, acc);

  if (wrole) dx_w_store(S.w[0], st, pre, mu, L);
  else act_store(S.x[0], st, pre);
  __syncthreads();

  for (uint32_t nb = 0; nb + 1 < nnb; ++nb) {
    const int buf = nb & 1;
    if (wrole) dx_w_load(ws, (nb + 1) * BK, pre);
    else act_load(yr, (uint32_t)N, (nb + 1) * BK, st, pre);
    mma_stage(S.w[buf], S.x[buf], wf, wmt, lr, lg, acc);
    if (wrole) dx_w_store(S.w[buf ^ 1], st, pre, mu, L);
    else act_store(S.x[buf ^ 1], st, pre);
    __syncthreads();
  }
  mma_stage(S.w[(nnb - 1) & 1], S.x[(nnb - 1) & 1], wf, wmt, lr, lg, acc);
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
