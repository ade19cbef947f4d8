// Weight-streaming forward for few tokens (M <= 16) over large weights: Y = X w_hat^T +
// s (X A^T) B^T, one launch.  Used when d_in is a multiple of 256 and d_out * d_in >= 32M;
// smaller weights take the kernel in gemv.hip, whose set-up per workgroup is cheaper.
//
// At small batch the layer is bound by reading the 4-bit weights from HBM ("QLoRA --
// Fine-Tuning a 65B Model on One GPU", "Pitfalls": small-batch generation is memory-bound
// and 4 bits leave less to read).  Each weight is decoded once, on chip, from its 4-bit code
// ("QLoRA: Quantize Base Weights to 4-Bit", Section 3) and multiplied on the MFMA units.
//
// Work split.  A workgroup owns 256 weight rows (8 wavefronts x one 32-row MFMA tile) and a
// contiguous range of 64-weight blocks (one of `ksplit` ranges).  At the start it stages in
// LDS what every wavefront shares: the activations of the range, the E4M3 block constants and
// second-level scales of its rows, and the byte-pair decode table.  The 4-bit codes never
// touch LDS: each wavefront streams its own rows straight into registers, kDepth chunks of
// kCB blocks in flight, with no barrier in the loop.  Without a reduction split, row group g
// walks its chunks starting at chunk g (mod their count), so that the workgroups do not all
// read the same column offset at once.
//
// MFMA mapping (v_mfma_f32_32x32x16_bf16).  Lane (n = lane & 31, h = lane >> 5) loads the 16
// bytes [16 h, 16 h + 16) of block b of weight row n: 32 weights, four code words.  Step s
// of the block uses word s, so the four steps cover the block's 64 weights and every
// reduction index of a step lies in one block: the block constant c1_hat multiplies the
// 32x32 partial product once, in FP32.  A code byte holds weights e_i and e_{i+4} of its
// word; one LDS lookup per byte (a table of the 256 byte values, one copy per lane so that
// 64 lookups hit 64 banks) yields both as BF16, so the weights of a word arrive in the order
// e0 e4 e1 e5 e2 e6 e3 e7.  The activations are staged in that same order, which leaves the
// products unchanged.  The lookups of step t + 1 are issued before the MFMA of step t.
//
// Adapter.  T = X A^T is linear in the reduction range, so each workgroup forms the part of
// T over its own range with 16x16x32 MFMAs (wavefront w takes the 32-index step w of every
// chunk, for every 16-rank tile), applies B to it for its rows, and adds that to its partial
// output.
//
// Grouped launch.  Linears that read the same activations (the q, k and v projections of a
// decoder layer, or its gate and up projections) can run as one launch: their row groups
// are numbered one after the other, each workgroup first finds the linear its row group
// belongs to, and from there on works as in a single launch.  One launch pays the start-up
// and the split-K hand-off once for the whole group instead of once per linear.
//
// Split-K reduction.  With ksplit > 1 each workgroup writes an FP32 partial; the last
// workgroup of a row group to finish (a device-scope arrival counter per row group of the
// launch, in the caller's workspace; that workgroup resets it to zero) sums the partials in
// a fixed order and writes BF16 Y (and T for the backward).  Calls that share a workspace
// must not overlap; calls with separate workspaces may.  The partials travel through memory with system-scope
// (cache-bypassing) stores and loads: the writer waits for its stores to complete before
// advancing the counter, so the reader needs no cache write-back fence.
#include "qlora_device.h"
#include "qlora_host.h"

namespace qlora {

namespace {

typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kRows = kWaves * 32;       // weight rows per workgroup
constexpr int kCB = 4;                   // blocks per chunk
constexpr int kLutBytes = 256 * 64 * 4;  // byte-pair table, one copy per lane
constexpr int kMaxR = 128;
constexpr int kRegion = 87 * 1024;       // activations, block constants, scales (then the T sums)
constexpr int kC8Loads = 24;             // staged block-constant dwords per thread, at most
constexpr int kSumU = 16;                // partials loaded together in the split-K sum
constexpr uint32_t kTag = 0x10000u;      // marks a handed-over word (tag | bf16)
constexpr int kMaxHandP = 8;             // reduction pieces of 4096 per producer lane (K <= 32768)

// Workgroup barrier that waits for this wavefront's LDS accesses only (lgkmcnt), so global
// loads in flight stay in flight across it.  Every barrier here orders LDS traffic between
// the wavefronts; none orders global memory.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("s_barrier" ::: "memory");
}

__device__ __forceinline__ f32x16_t mfma32(const bf16x8_t& a, const bf16x8_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// OCP E4M3 byte -> FP32 without a branch: normal (exponent field e > 0) 2^(e-7) (1 + m/8),
// subnormal m 2^-9.
__device__ __forceinline__ float e4m3_value(uint32_t b) {
  const float nrm = __uint_as_float(((b & 0x7Fu) << 20) + 0x3C000000u);
  const float sub = (float)(b & 7u) * 0.001953125f;
  const float v = (b & 0x78u) ? nrm : sub;
  return (b & 0x80u) ? -v : v;
}

// 8 BF16 values e0..e7 (4 dwords of pairs) reordered to e0 e4 e1 e5 e2 e6 e3 e7.
__device__ __forceinline__ uint4 pair_order(uint4 v) {
  return make_uint4(__builtin_amdgcn_perm(v.z, v.x, 0x05040100u), __builtin_amdgcn_perm(v.z, v.x, 0x07060302u),
                    __builtin_amdgcn_perm(v.w, v.y, 0x05040100u), __builtin_amdgcn_perm(v.w, v.y, 0x07060302u));
}

// The 8 weights of code word w in pair order, looked up in the byte-pair table (at LDS
// address 0): the address of byte p is (byte << 8) | (lane * 4).
__device__ __forceinline__ void decode_pairs(uint32_t w, uint32_t lane4, const uint8_t* lut, uint32_t out[4]) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t addr = __builtin_amdgcn_perm(w, lane4, 0x0C0C0400u | ((4u + p) << 8));
    out[p] = *reinterpret_cast<const uint32_t*>(lut + addr);
  }
}

struct StreamArgs {
  const uint8_t* codes;
  const uint8_t* code8;
  const float* c2s;
  const float* mu;
  const uint16_t* X;
  const uint16_t* A;
  const uint16_t* B;
  uint16_t* Y;
  uint16_t* T_save;
  float* part;   // [ksplit][M][N]
  float* tpart;  // [ksplit][M][r]
  unsigned int* counters;  // [row groups of the launch], zero between calls
  uint32_t* words;         // handed-over T: [row groups of the launch][r] (tag | bf16(s T)), zero between calls
  int32_t nprod;           // workgroups that also form a column of T (the first ones dispatched)
  int64_t N, K;
  int32_t M, r;
  float s;
  int32_t ksplit;
  int32_t nbs;     // blocks per split (a multiple of kCB)
  int32_t nchunk;  // chunks per split, a multiple of kDepth (chunks past the range add zeros)
  int32_t xpitch;  // bytes per staged activation row
  int32_t c8pitch; // bytes per staged row of block constants (nbs + 4)
  int32_t c8off;   // region offset of the block constants
  int32_t c2off;   // region offset of the second-level scales
  int32_t c2max;   // scales staged per workgroup
};

// Per-linear operands of a grouped launch (count <= kMaxLin linears of d_out a multiple of
// kRows, sharing d_in, M, r and the codebook).  Row group g of the launch belongs to linear i
// for gstart[i] <= g < gstart[i + 1].
constexpr int kMaxLin = 4;
struct StreamGroup {
  const uint8_t* codes[kMaxLin];
  const uint8_t* code8[kMaxLin];
  const float* c2s[kMaxLin];
  const float* mu[kMaxLin];
  const uint16_t* A[kMaxLin];
  const uint16_t* B[kMaxLin];
  uint16_t* Y[kMaxLin];
  uint16_t* T_save[kMaxLin];
  int32_t gstart[kMaxLin + 1];
  int32_t count;
};
struct NoGroup {};
template <bool MULTI> struct GroupArg { typedef NoGroup type; };
template <> struct GroupArg<true> { typedef StreamGroup type; };

struct Smem {
  uint8_t lut[kLutBytes];  // first, so that its LDS address is 0
  uint8_t region[kRegion];
  float t[16][kMaxR + 4];
  float tp[kWaves];  // a T producer's per-wavefront parts
  unsigned int last;
};

// Registers of one chunk between issue and use.
template <int RT16>
struct Chunk {
  uint4 cw[kCB];     // codes of block i: bytes [16 h, 16 h + 16) of row n
  uint4 av[RT16];    // adapter rows 16 k + (lane & 15), this wavefront's 32-index step
};

// RT16: 16-wide rank tiles (r <= 16 RT16).  NQ: accumulator registers kept (1 for M = 1,
// where only row 0 of the 32x32 product is live; 8 for M <= 16).  K is a multiple of 256, so
// a chunk's four E4M3 bytes form one aligned word and share one second-level scale.
// HAND (M = 1 only): T is not formed in the loop.  The first count r workgroups in dispatch
// order each also form one column j of T = x A^T of one linear over the whole reduction
// (8 products per lane and piece of 4096, a fixed-order DPP sum per wavefront, then the
// wavefronts in order) while their first chunks land, and write bf16(s T) with a tag into
// the word block of every row group of that linear in the workspace head.  Row groups take
// the adapter term in split 0 only: after the loop, each wavefront reads its row group's
// words (bounded wait), applies them to B on MFMA and adds the result; the words are cleared
// after the outputs.  Producers wait on nothing before they publish and are dispatched
// first, so no reader waits on a workgroup that has not started.
template <int RT16, int NQ, int kDepth, bool MULTI, bool HAND>
__global__ __launch_bounds__(kThreads) void k_gemv_stream(StreamArgs a, Lut L, typename GroupArg<MULTI>::type G) {
  __shared__ Smem sm;
  const uint8_t* const sLut = sm.lut;
  uint8_t* const sR = sm.region;
  auto& sT = sm.t;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5, l16 = lane & 15, g = lane >> 4;
  // Nt, pgrp: rows and row group of the launch (partials, counters); N, grp: of the linear
  const int64_t Nt = a.N, K = a.K;
  const int M = a.M;
  const int64_t nb_row = K / kBlock1;
  const int64_t pgrp = blockIdx.x;
  const int ks = blockIdx.y;
  int64_t N = Nt, grp = pgrp;
  float* tpart = a.tpart;
  const uint8_t* w_codes = a.codes;
  const uint8_t* w_code8 = a.code8;
  const float* w_c2s = a.c2s;
  const float* w_mu = a.mu;
  const uint16_t* l_A = a.A;
  const uint16_t* l_B = a.B;
  uint16_t* o_Y = a.Y;
  uint16_t* o_T = a.T_save;
  if constexpr (MULTI) {
    int li = 0;
#pragma unroll
    for (int i = 1; i < kMaxLin; ++i)
      if (i < G.count && (int)blockIdx.x >= G.gstart[i]) li = i;
    w_codes = G.codes[li];
    w_code8 = G.code8[li];
    w_c2s = G.c2s[li];
    w_mu = G.mu[li];
    l_A = G.A[li];
    l_B = G.B[li];
    o_Y = G.Y[li];
    o_T = G.T_save[li];
    N = (int64_t)(G.gstart[li + 1] - G.gstart[li]) * kRows;
    grp = pgrp - G.gstart[li];
    tpart += (int64_t)li * a.ksplit * M * a.r;
  }
  // T producer role (HAND): column pj of linear pli
  const int64_t lin = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;  // dispatch order
  const bool producer = HAND && lin < a.nprod;
  const int pj = producer ? (int)(lin % a.r) : 0, pli = producer ? (int)(lin / a.r) : 0;
  const rsrc_t rx = make_rsrc(a.X, (int64_t)M * K * 2);
  uint4 hx[HAND ? kMaxHandP : 1], ha[HAND ? kMaxHandP : 1];
  if (HAND && producer) {
    const uint16_t* pA = a.A;
    if constexpr (MULTI) pA = G.A[pli];
    const rsrc_t rpa = make_rsrc(pA + (int64_t)pj * K, K * 2);
#pragma unroll
    for (int p = 0; p < (HAND ? kMaxHandP : 1); ++p) {
      const int64_t k = 4096 * p + 8 * (64 * wave + lane);
      hx[p] = bload16(rx, k < K ? (uint32_t)(k * 2) : kOOB);
      ha[p] = bload16(rpa, k < K ? (uint32_t)(k * 2) : kOOB);
    }
  }
  const int64_t b0 = (int64_t)ks * a.nbs;
  const int64_t b1 = (b0 + a.nbs < nb_row) ? b0 + a.nbs : nb_row;
  const int64_t row0 = grp * kRows;
  const int64_t n = row0 + 32 * wave + l32;  // this lane's weight row
  const float mu = w_mu[0];

  const rsrc_t rc = make_rsrc(w_codes, N * (K / 2));
  const rsrc_t r8 = make_rsrc(w_code8, N * nb_row);
  const rsrc_t r2 = make_rsrc(w_c2s, ((N * nb_row + 255) / 256) * 4);
  const rsrc_t ra = make_rsrc(l_A, (int64_t)a.r * K * 2);
  const rsrc_t rb = make_rsrc(l_B, N * a.r * 2);

  const uint32_t code_row = n < N ? (uint32_t)(n * (K / 2)) + 16u * h : kOOB;
  // first second-level group touched by this workgroup
  const int64_t g0 = (row0 * nb_row + b0) >> 8;

  // chunks holding blocks of this range; the rest of nchunk only pads the unrolled loop.
  // Without a reduction split every workgroup walks the whole row, and all of them would read
  // the same reduction offset (their codes at the same column, the same A rows) at the same
  // time; so workgroup `grp` starts at its chunk grp mod nreal and wraps around (a fixed
  // order per row group, the same in a grouped launch).
  const int nreal = (int)(((b1 > b0 ? b1 - b0 : 0) + kCB - 1) / kCB);
  const int rot = (a.ksplit == 1 && nreal > 0) ? (int)(grp % nreal) : 0;
  // (ci + rot) mod nreal without a division: both terms are below nreal
  auto chunk_of = [&](int ci) { return ci < nreal ? (ci + rot >= nreal ? ci + rot - nreal : ci + rot) : ci; };
  auto issue = [&](int ci, Chunk<RT16>& C) {
    const int64_t bc = b0 + (int64_t)chunk_of(ci) * kCB;
#pragma unroll
    for (int i = 0; i < kCB; ++i) {
      const bool ok = bc + i < b1 && code_row != kOOB;
      C.cw[i] = bload16(rc, ok ? code_row + (uint32_t)((bc + i) * 32) : kOOB);
    }
    // adapter: rows 16 k + l16, reduction indices 64 bc + 32 wave + 8 g .. + 8
    if constexpr (!HAND) {
#pragma unroll
      for (int k = 0; k < RT16; ++k) {
        const int j = 16 * k + l16;
        const bool ok = bc < b1 && j < a.r;
        C.av[k] = bload16(ra, ok ? (uint32_t)(((int64_t)j * K + bc * 64 + 32 * wave + 8 * g) * 2) : kOOB);
      }
    }
  };

  // ---- staging.  Issue order: the codes of chunk 0 (needed first, from HBM), the block
  // constants, activations and scales, then the next chunks of codes and the B rows, which
  // stay in flight while the staged data is written.
  Chunk<RT16> C[kDepth];
  issue(0, C[0]);
  // block constants of the range: dword d of the staged [kRows][c8pitch] block is row d / c8w,
  // bytes 4 (d % c8w) .. + 3 of the row's range (the last dword of a row is padding).  The
  // row and column of d = u kThreads + tid advance by the quotient and remainder of kThreads
  // / c8w from pass to pass (one division per thread, not one per pass: an integer division
  // is a few dozen instructions, and they delayed the issue of every later load).
  const int c8w = a.c8pitch / 4;
  const int dwords = kRows * c8w;
  const int c8q = kThreads / c8w, c8r = kThreads - c8q * c8w;
  uint32_t c8v[kC8Loads];
  {
    // 32-bit operands (rows below 2^22, the range below 2^26 blocks) and no short-circuit,
    // so that the test and the offset are selects, not branches
    const int rows_left = (int)(N - row0), span = (int)(b1 - b0);
    const uint32_t c8base = (uint32_t)(row0 * nb_row + b0), nbr = (uint32_t)nb_row;
    int row = tid / c8w, cd = tid - (tid / c8w) * c8w;
#pragma unroll
    for (int u = 0; u < kC8Loads; ++u) {
      if (u * kThreads < dwords) {  // uniform: only the passes that hold staged dwords
        const int d = u * kThreads + tid;
        const bool ok = (d < dwords) & (row < rows_left) & (4 * cd < span);
        c8v[u] = bload4(r8, ok ? c8base + (uint32_t)row * nbr + 4u * (uint32_t)cd : kOOB);
      }
      row += c8q;
      cd += c8r;
      if (cd >= c8w) {
        cd -= c8w;
        ++row;
      }
    }
  }
  // activations of this range, pair-ordered: rows 0..M-1 then a zero row.  (M + 1) rows of
  // nchunk * kCB * 128 bytes are at most 4096 pieces of 16 bytes: one batch of 8 per thread.
  // Item i = u kThreads + tid is piece i % pieces of row i / pieces, advanced per pass as above;
  // xo[u] keeps its LDS offset for the staging writes.
  const int pieces = a.nchunk * kCB * 8;
  const int items = (M + 1) * pieces;
  const int xq = kThreads / pieces, xr = kThreads - xq * pieces;
  uint4 xv[8];
  int xo[8];
  {
    const int kspan = (int)(64 * (b1 - b0));  // reduction indices of the range
    const uint32_t xbase = (uint32_t)(b0 * 128), xrow = (uint32_t)(2 * K);
    int m = tid / pieces, pc = tid - (tid / pieces) * pieces;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      xo[u] = m * a.xpitch + 16 * pc;
      if (u * kThreads < items) {  // uniform: only the passes that hold pieces
        const int i = u * kThreads + tid;
        const bool ok = (i < items) & (m < M) & (8 * pc < kspan);
        xv[u] = bload16(rx, ok ? (uint32_t)m * xrow + xbase + 16u * (uint32_t)pc : kOOB);
      }
      m += xq;
      pc += xr;
      if (pc >= pieces) {
        pc -= pieces;
        ++m;
      }
    }
  }
  const uint32_t c2v = bload4(r2, tid < a.c2max ? (uint32_t)((g0 + tid) * 4) : kOOB);

#pragma unroll
  for (int d = 1; d < kDepth - 1; ++d) issue(d, C[d]);

  // B rows for the adapter up-projection (r <= 32 prefetched; larger r loaded at the end)
  uint4 bpre[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int j = 16 * u + 8 * h;
    const bool ok = (a.r % 8) == 0 && j < a.r && n < N;
    bpre[u] = bload16(rb, ok ? (uint32_t)((n * a.r + j) * 2) : kOOB);
  }

  // byte-pair table: pass i, lane l writes 4 copies of entry 32 i + 4 wave + l / 16
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t e = 32u * i + 4u * wave + (lane >> 4);
    uint32_t d[4];
    decode8((e & 15u) | ((e >> 4) << 8), L, d);
    *reinterpret_cast<uint4*>(sm.lut + e * 256 + (lane & 15) * 16) = make_uint4(d[0], d[0], d[0], d[0]);
  }
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int i = u * kThreads + tid;
    if (u * kThreads < items && i < items) *reinterpret_cast<uint4*>(sR + xo[u]) = pair_order(xv[u]);
  }
  if (tid < a.c2max) reinterpret_cast<float*>(sR + a.c2off)[tid] = __uint_as_float(c2v);
#pragma unroll
  for (int u = 0; u < kC8Loads; ++u) {
    const int d = u * kThreads + tid;
    if (u * kThreads < dwords && d < dwords) reinterpret_cast<uint32_t*>(sR + a.c8off)[d] = c8v[u];
  }
  if (HAND && producer) {  // this wavefront's part of T[0][pj]
    float d = 0.f;
#pragma unroll
    for (int p = 0; p < (HAND ? kMaxHandP : 1); ++p) {
      const uint32_t xw[4] = {hx[p].x, hx[p].y, hx[p].z, hx[p].w}, aw[4] = {ha[p].x, ha[p].y, ha[p].z, ha[p].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        d = fmaf(bf16lo_to_f32(xw[e]), bf16lo_to_f32(aw[e]), d);
        d = fmaf(bf16hi_to_f32(xw[e]), bf16hi_to_f32(aw[e]), d);
      }
    }
    const float t = wave_sum(d);
    if (lane == 0) sm.tp[wave] = t;
  }
  lds_barrier();
  if (HAND && producer) {  // publish column pj to every row group of linear pli
    float t = sm.tp[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) t += sm.tp[w];
    uint16_t* pT = a.T_save;
    int gb = 0, ge = (int)gridDim.x;
    if constexpr (MULTI) {
      pT = G.T_save[pli];
      gb = G.gstart[pli];
      ge = G.gstart[pli + 1];
    }
    if (tid == 0 && pT) pT[pj] = (uint16_t)(pack_bf16x2(t, 0.f) & 0xFFFFu);
    const uint32_t word = kTag | (pack_bf16x2(a.s * t, 0.f) & 0xFFFFu);
    for (int q = gb + tid; q < ge; q += kThreads)
      __hip_atomic_store(a.words + (int64_t)q * a.r + pj, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }

  const uint32_t lane4 = (uint32_t)lane * 4u;
  // activation rows of this lane (rows >= M read the zero row): 32x32 operand and 16x16 operand
  const uint8_t* const xrow = sR + (l32 < M ? l32 : M) * a.xpitch + 64 * h;
  const uint8_t* const xrow16 = sR + (l16 < M ? l16 : M) * a.xpitch + 64 * wave + 16 * g;
  const uint8_t* const c8row = sR + a.c8off + (32 * wave + l32) * a.c8pitch;
  const float* const c2l = reinterpret_cast<const float*>(sR + a.c2off);

  float acc[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) acc[q] = 0.f;
  f32x4_t tacc[RT16];
#pragma unroll
  for (int k = 0; k < RT16; ++k) tacc[k] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int step, const Chunk<RT16>& Cc) {
    const int ci = chunk_of(step);
    const int64_t bc = b0 + (int64_t)ci * kCB;
    const uint8_t* xc = xrow + ci * kCB * 128;
    float cs[kCB];
    const uint32_t w8 = *reinterpret_cast<const uint32_t*>(c8row + 4 * ci);
    const float c2 = c2l[((n * nb_row + bc) >> 8) - g0];
#pragma unroll
    for (int i = 0; i < kCB; ++i) cs[i] = __fadd_rn(__fmul_rn(e4m3_value((w8 >> (8 * i)) & 0xFFu), c2), mu);
    // step t = 4 i + s: block i, word s.  The lookups and the activation read of step t + 1
    // are issued before the MFMA of step t, so their LDS latency overlaps it.
    auto word = [&](int t) {
      const uint4& v = Cc.cw[t / 4];
      return (t % 4 == 0) ? v.x : (t % 4 == 1) ? v.y : (t % 4 == 2) ? v.z : v.w;
    };
    uint32_t w[2][4];
    uint4 xv2[2];
    decode_pairs(word(0), lane4, sLut, w[0]);
    xv2[0] = *reinterpret_cast<const uint4*>(xc);
    f32x16_t p = {};
#pragma unroll
    for (int t = 0; t < 4 * kCB; ++t) {
      const int cur = t & 1;
      if (t + 1 < 4 * kCB) {
        decode_pairs(word(t + 1), lane4, sLut, w[cur ^ 1]);
        xv2[cur ^ 1] = *reinterpret_cast<const uint4*>(xc + ((t + 1) / 4) * 128 + 16 * ((t + 1) % 4));
      }
      p = mfma32(as_bf16x8(xv2[cur]), as_bf16x8(w[cur]), (t % 4 == 0) ? f32x16_t{} : p);
      if (t % 4 == 3) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) acc[q] = fmaf(cs[t / 4], p[q], acc[q]);
      }
    }
    // adapter: this wavefront's 32-index step of the chunk, every rank tile
    if constexpr (!HAND) {
      const bf16x8_t xt = as_bf16x8(*reinterpret_cast<const uint4*>(xrow16 + ci * kCB * 128));
#pragma unroll
      for (int k = 0; k < RT16; ++k) tacc[k] = mfma16x16x32(xt, as_bf16x8(pair_order(Cc.av[k])), tacc[k]);
    }
  };

  for (int ci0 = 0; ci0 < a.nchunk; ci0 += kDepth) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      if (kDepth > 1) issue(ci0 + d + kDepth - 1, C[(d + kDepth - 1) % kDepth]);
      if (ci0 + d < nreal) compute(ci0 + d, C[d]);
    }
  }

  // ---- T over this range: sum the wavefronts' parts (without HAND)
  if constexpr (!HAND) {
    lds_barrier();  // every wavefront is done with the staged region
    float* sred = reinterpret_cast<float*>(sR);  // [kWaves][RT16][64][4]
#pragma unroll
    for (int k = 0; k < RT16; ++k)
      *reinterpret_cast<f32x4_t*>(sred + ((wave * RT16 + k) * 64 + lane) * 4) = tacc[k];
    lds_barrier();
    for (int i = tid; i < M * a.r; i += kThreads) {
      const int m = i / a.r, j = i % a.r;
      const int k = j / 16, ln = (j % 16) + 16 * (m / 4), v = m % 4;  // D[m = 4 (lane >> 4) + v][j = lane & 15]
      float sum = 0.f;
      for (int w = 0; w < kWaves; ++w) sum += sred[((w * RT16 + k) * 64 + ln) * 4 + v];
      sT[m][j] = sum;
    }
    lds_barrier();
  }

  // ---- adapter up-projection: rows n of this wavefront, with this range's T, or (HAND) with
  // the handed-over T in split 0 only
  uint32_t* const mine = HAND ? a.words + pgrp * a.r : nullptr;  // this row group's words
  if (!HAND || ks == 0) {
    f32x16_t up = {};
#pragma unroll
    for (int u = 0; u < kMaxR / 16; ++u) {
      if (16 * u >= a.r) break;
      const int j0 = 16 * u + 8 * h;
      uint32_t tv[4];
      if constexpr (HAND) {
        // bounded wait (about 2^20 polls): should the words never arrive, the outputs become
        // NaN instead of the wavefront spinning forever
        const bool live = l32 == 0;  // token row 0 of the A operand
        uint32_t tw[8];
        bool ready = false;
        for (int it = 0; !ready && it < (1 << 20); ++it) {
          if (it) __builtin_amdgcn_s_sleep(2);
#pragma unroll
          for (int i = 0; i < 8; ++i)
            tw[i] = (live && j0 + i < a.r) ? __hip_atomic_load(mine + j0 + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM)
                                           : kTag;
          ready = true;
#pragma unroll
          for (int i = 0; i < 8; ++i) ready = ready && (tw[i] & 0xFFFF0000u) == kTag;
        }
        if (!ready) {
#pragma unroll
          for (int i = 0; i < 8; ++i) tw[i] = kTag | 0x7FC0u;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) tv[e] = live ? ((tw[2 * e] & 0xFFFFu) | (tw[2 * e + 1] << 16)) : 0u;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float lo = (l32 < M && j0 + 2 * e < a.r) ? a.s * sT[l32][j0 + 2 * e] : 0.f;
          const float hi = (l32 < M && j0 + 2 * e + 1 < a.r) ? a.s * sT[l32][j0 + 2 * e + 1] : 0.f;
          tv[e] = pack_bf16x2(lo, hi);
        }
      }
      uint4 bw;
      if (u < 2 && (a.r % 8) == 0) {
        bw = bpre[u < 2 ? u : 0];  // u is a compile-time index here
      } else {
        uint32_t e8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          e8[e] = __builtin_amdgcn_raw_buffer_load_b16(rb, (j0 + e < a.r && n < N) ? (int)((n * a.r + j0 + e) * 2) : (int)kOOB, 0, 0);
        bw = make_uint4((e8[0] & 0xFFFFu) | (e8[1] << 16), (e8[2] & 0xFFFFu) | (e8[3] << 16),
                        (e8[4] & 0xFFFFu) | (e8[5] << 16), (e8[6] & 0xFFFFu) | (e8[7] << 16));
      }
      up = mfma32(as_bf16x8(tv), as_bf16x8(bw), up);
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q) acc[q] += up[q];
  }

  // ---- output: register 4 q + v of lane (n, h) holds row m = 8 q + 4 h + v of column n
  if (a.ksplit == 1) {
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int m = 8 * (q / 4) + 4 * h + (q % 4);
      if (m < M && n < N) o_Y[(int64_t)m * N + n] = (uint16_t)(pack_bf16x2(acc[q], 0.f) & 0xFFFFu);
    }
    if (!HAND && o_T && grp == 0) {
      for (int i = tid; i < M * a.r; i += kThreads)
        o_T[i] = (uint16_t)(pack_bf16x2(sT[i / a.r][i % a.r], 0.f) & 0xFFFFu);
    }
    if (HAND) {  // every wavefront has read the words: clear them for the next call
      lds_barrier();
      for (int i = tid; i < a.r; i += kThreads)
        __hip_atomic_store(mine + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
    return;
  }
  const int64_t pn = pgrp * kRows + 32 * wave + l32;  // this lane's column of the launch's partials
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int m = 8 * (q / 4) + 4 * h + (q % 4);
    if (m < M && n < N)
      __hip_atomic_store(a.part + ((int64_t)ks * M + m) * Nt + pn, acc[q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }
  if (!HAND && grp == 0) {
    for (int i = tid; i < M * a.r; i += kThreads)
      __hip_atomic_store(tpart + (int64_t)ks * M * a.r + i, sT[i / a.r][i % a.r], __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_SYSTEM);
  }
  // every partial store of this workgroup has completed before its counter increment
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (HAND && ks == 0) {  // every wavefront has read the words: clear them for the next call
    for (int i = tid; i < a.r; i += kThreads)
      __hip_atomic_store(mine + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }
  if (tid == 0) {
    const unsigned int old = __hip_atomic_fetch_add(&a.counters[pgrp], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sm.last = (old + 1u == (unsigned int)a.ksplit) ? 1u : 0u;
    if (sm.last) __hip_atomic_store(&a.counters[pgrp], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!sm.last) return;
  // last workgroup of this row group: fixed-order sum of the partials
  auto sum_published = [&](const float* p, int32_t cnt, int64_t stride) {
    float sum = 0.f;
    for (int32_t k0 = 0; k0 < cnt; k0 += kSumU) {
      float v[kSumU];
#pragma unroll
      for (int u = 0; u < kSumU; ++u)
        v[u] = (k0 + u < cnt) ? __hip_atomic_load(p + (int64_t)(k0 + u) * stride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) : 0.f;
#pragma unroll
      for (int u = 0; u < kSumU; ++u) sum += v[u];
    }
    return sum;
  };
  const int64_t nrows = (row0 + kRows <= N) ? kRows : N - row0;
  for (int64_t i = tid; i < (int64_t)M * nrows; i += kThreads) {
    // 32-bit, by a shift for a whole group (a 64-bit division is a long sequence, in the tail)
    const int nr = (int)nrows, ii = (int)i;
    const int m = nr == kRows ? (int)((unsigned)ii / (unsigned)kRows) : (int)((unsigned)ii / (unsigned)nr);
    const int nn = ii - m * nr;
    o_Y[m * N + row0 + nn] =
        (uint16_t)(pack_bf16x2(sum_published(a.part + m * Nt + pgrp * kRows + nn, a.ksplit, (int64_t)M * Nt), 0.f) &
                   0xFFFFu);
  }
  if (!HAND && o_T && grp == 0) {
    for (int i = tid; i < M * a.r; i += kThreads)
      o_T[i] = (uint16_t)(pack_bf16x2(sum_published(tpart + i, a.ksplit, (int64_t)M * a.r), 0.f) & 0xFFFFu);
  }
}

// LDS region use of a split of nbs blocks (nchunk chunks) for M rows of activations.
struct RegionUse {
  int32_t xpitch, c8pitch, c8off, c2off, c2max, c8dw, total;
};
RegionUse region_use(int64_t nb_row, int64_t M, int64_t nbs, int64_t nchunk) {
  RegionUse u{};
  u.xpitch = (int32_t)(nchunk * kCB * 128 + 16);
  u.c8pitch = (int32_t)(nbs + 4);
  u.c8off = (int32_t)(((M + 1) * u.xpitch + 15) / 16 * 16);
  u.c2off = (int32_t)((u.c8off + kRows * u.c8pitch + 15) / 16 * 16);
  u.c8dw = kRows * u.c8pitch / 4;
  // groups touched by kRows rows over nbs blocks: at most (kRows - 1) nb_row / 256 + 2
  u.c2max = (int32_t)(((kRows - 1) * nb_row + nbs) / 256 + 2);
  u.total = u.c2off + 4 * u.c2max;
  return u;
}

// Chunks in flight per wavefront: three where registers allow (r <= 32), else two.  Plans
// whose ranges are single chunks run with one (no prefetch to issue).
int stream_depth(int32_t r) { return r <= 32 ? 3 : 2; }

}  // namespace

GemvPlan gemv_stream_plan(int64_t N, int64_t K, int64_t M, int32_t r) {
  GemvPlan p{};
  const int kDepth = stream_depth(r);
  p.groups = (N + kRows - 1) / kRows;
  const int64_t nb_row = K / kBlock1;
  auto chunks_of = [&](int64_t nbs) { return ((nbs / kCB + kDepth - 1) / kDepth) * kDepth; };
  auto nbs_of = [&](int64_t ks) { return ((nb_row + ks - 1) / ks + kCB - 1) / kCB * kCB; };
  // One workgroup per CU (256 CUs).  Estimated time of a split: rounds of workgroups x (its
  // chunks + a fixed cost of about three chunks for the first loads and the reduction).
  constexpr int64_t kFixed = 3;
  int64_t best_ks = 0, best_cost = 0;
  for (int64_t ks = 1; ks <= nb_row && ks <= 65535; ++ks) {
    const int64_t nbs = nbs_of(ks);
    const int64_t used = (nb_row + nbs - 1) / nbs;  // non-empty ranges
    if (used != ks) continue;
    const RegionUse u = region_use(nb_row, M, nbs, chunks_of(nbs));
    if (u.total > kRegion || (M + 1) * chunks_of(nbs) * kCB * 8 > 8 * kThreads || u.c2max > kThreads ||
        u.c8dw > kC8Loads * kThreads)
      continue;
    const int64_t wgs = p.groups * ks;
    const int64_t cost = ((wgs + 255) / 256) * (nbs / kCB + kFixed);
    if (best_ks == 0 || cost < best_cost) {
      best_ks = ks;
      best_cost = cost;
    }
  }
  p.ksplit = (int32_t)best_ks;
  if (best_ks == 0) return p;  // no split fits the staging limits: the shape is not streamed
  p.nbs = (int32_t)nbs_of(best_ks);
  p.nchunk = p.nbs <= kCB ? 1 : (int32_t)chunks_of(p.nbs);
  p.xpitch = region_use(nb_row, M, p.nbs, p.nchunk).xpitch;
  return p;
}

bool gemv_stream_fits(int64_t N, int64_t K, int64_t M, int32_t r) {
  if (M < 1 || M > 16 || r < 1 || r > kMaxR || K % 256 != 0 || N * K < (int64_t(32) << 20)) return false;
  return gemv_stream_plan(N, K, M, r).ksplit >= 1;
}

bool gemv_stream_group_fits(int count, const int64_t* N, int64_t K, int64_t M, int32_t r) {
  if (count < 2 || count > kMaxLin) return false;
  int64_t Nt = 0;
  for (int i = 0; i < count; ++i) {
    if (N[i] < 1 || N[i] % kRows != 0) return false;
    Nt += N[i];
  }
  return Nt / kRows <= 65536 && gemv_stream_fits(Nt, K, M, r);
}

namespace {

// One launch over `count` linears (count == 1: the single-linear kernel, without the group
// table in its arguments).
hipError_t stream_launch(int count, const StreamLinear* lins, int64_t K, const uint16_t* X, int64_t M, int32_t r,
                         float s, float* part, float* tpart, unsigned int* counters, const Nf4Tables& T,
                         hipStream_t st) {
  if (count < 1 || count > kMaxLin || M < 1 || M > 16 || r < 1 || r > kMaxR) return hipErrorInvalidValue;
  int64_t Nt = 0;
  for (int i = 0; i < count; ++i) {
    if (count > 1 && lins[i].N % kRows != 0) return hipErrorInvalidValue;
    Nt += lins[i].N;
  }
  const GemvPlan p = gemv_stream_plan(Nt, K, M, r);
  const int64_t nb_row = K / kBlock1;
  const RegionUse u = region_use(nb_row, M, p.nbs, p.nchunk);
  if (p.ksplit < 1 || u.total > kRegion || (M + 1) * p.nchunk * kCB * 8 > 8 * kThreads || u.c2max > kThreads ||
      u.c8dw > kC8Loads * kThreads || nb_row % kCB != 0 || p.groups > 65536)
    return hipErrorInvalidValue;
  StreamArgs a;
  a.codes = reinterpret_cast<const uint8_t*>(lins[0].codes);
  a.code8 = lins[0].code8;
  a.c2s = lins[0].c2s;
  a.mu = lins[0].mu;
  a.X = X;
  a.A = lins[0].A;
  a.B = lins[0].B;
  a.Y = lins[0].Y;
  a.T_save = lins[0].T_save;
  a.part = part;
  a.tpart = tpart;
  a.counters = counters;
  // T handed over through words (M = 1): the words follow the counters in the head, and the
  // producers are row workgroups too, so there must be at least count r of those
  const int64_t woff = (p.groups + 63) / 64 * 64;
  const bool hand = M == 1 && K <= 4096 * kMaxHandP && (int64_t)count * r <= p.groups * p.ksplit &&
                    (size_t)(woff + p.groups * r) * 4 <= QLORA_WS_COUNTER_BYTES;
  a.words = hand ? reinterpret_cast<uint32_t*>(counters + woff) : nullptr;
  a.nprod = hand ? count * r : 0;
  a.N = Nt;
  a.K = K;
  a.M = (int32_t)M;
  a.r = r;
  a.s = s;
  a.ksplit = p.ksplit;
  a.nbs = p.nbs;
  a.nchunk = p.nchunk;
  a.xpitch = u.xpitch;
  a.c8pitch = u.c8pitch;
  a.c8off = u.c8off;
  a.c2off = u.c2off;
  a.c2max = u.c2max;
  Lut L;
  for (int w = 0; w < 4; ++w) {
    L.lo[w] = T.lut_lo[w];
    L.hi[w] = T.lut_hi[w];
  }
  StreamGroup G{};
  NoGroup none;
  G.count = count;
  G.gstart[0] = 0;
  for (int i = 0; i < count; ++i) {
    G.codes[i] = reinterpret_cast<const uint8_t*>(lins[i].codes);
    G.code8[i] = lins[i].code8;
    G.c2s[i] = lins[i].c2s;
    G.mu[i] = lins[i].mu;
    G.A[i] = lins[i].A;
    G.B[i] = lins[i].B;
    G.Y[i] = lins[i].Y;
    G.T_save[i] = lins[i].T_save;
    G.gstart[i + 1] = G.gstart[i] + (int32_t)(lins[i].N / kRows);
  }
  for (int i = count + 1; i <= kMaxLin; ++i) G.gstart[i] = G.gstart[count];
  dim3 grid((unsigned)p.groups, (unsigned)p.ksplit);
  LaunchTimer t(3, st);
#define QLORA_GEMV_GO1(RT16, NQ, D)                                                                                  \
  do {                                                                                                               \
    if (count > 1)                                                                                                   \
      hipExtLaunchKernelGGL((k_gemv_stream<RT16, NQ, D, true, false>), grid, dim3(kThreads), 0, st, t.start, t.stop, \
                            0, a, L, G);                                                                             \
    else                                                                                                             \
      hipExtLaunchKernelGGL((k_gemv_stream<RT16, NQ, D, false, false>), grid, dim3(kThreads), 0, st, t.start,       \
                            t.stop, 0, a, L, none);                                                                  \
  } while (0)
#define QLORA_GEMV_HAND1(D)                                                                                          \
  do {                                                                                                               \
    if (count > 1)                                                                                                   \
      hipExtLaunchKernelGGL((k_gemv_stream<1, 1, D, true, true>), grid, dim3(kThreads), 0, st, t.start, t.stop, 0, \
                            a, L, G);                                                                                \
    else                                                                                                             \
      hipExtLaunchKernelGGL((k_gemv_stream<1, 1, D, false, true>), grid, dim3(kThreads), 0, st, t.start, t.stop, 0, \
                            a, L, none);                                                                             \
  } while (0)
#define QLORA_GEMV_GO(RT16, NQ, D)            \
  do {                                        \
    if (p.nchunk == 1) QLORA_GEMV_GO1(RT16, NQ, 1); \
    else QLORA_GEMV_GO1(RT16, NQ, D);         \
  } while (0)
  if (hand) {
    if (p.nchunk == 1) QLORA_GEMV_HAND1(1);
    else if (stream_depth(r) == 3) QLORA_GEMV_HAND1(3);
    else QLORA_GEMV_HAND1(2);
  } else if (M == 1) {
    if (r <= 16) QLORA_GEMV_GO(1, 1, 3);
    else if (r <= 32) QLORA_GEMV_GO(2, 1, 3);
    else if (r <= 64) QLORA_GEMV_GO(4, 1, 2);
    else QLORA_GEMV_GO(8, 1, 2);
  } else {
    if (r <= 16) QLORA_GEMV_GO(1, 8, 3);
    else if (r <= 32) QLORA_GEMV_GO(2, 8, 3);
    else if (r <= 64) QLORA_GEMV_GO(4, 8, 2);
    else QLORA_GEMV_GO(8, 8, 2);
  }
#undef QLORA_GEMV_GO
#undef QLORA_GEMV_GO1
#undef QLORA_GEMV_HAND1
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_stream(const uint32_t* codes, const uint8_t* code8, const float* c2s,
                              const float* mu, int64_t N, int64_t K, const uint16_t* X, int64_t M,
                              const uint16_t* A, const uint16_t* B, int32_t r, float s, uint16_t* Y,
                              uint16_t* T_save, float* part, float* tpart, unsigned int* counters,
                              const Nf4Tables& T, hipStream_t st) {
  const StreamLinear one{codes, code8, c2s, mu, N, A, B, Y, T_save};
  return stream_launch(1, &one, K, X, M, r, s, part, tpart, counters, T, st);
}

hipError_t launch_gemv_stream_group(int count, const StreamLinear* lins, int64_t K, const uint16_t* X, int64_t M,
                                    int32_t r, float s, float* part, float* tpart, unsigned int* counters,
                                    const Nf4Tables& T, hipStream_t st) {
  if (count < 2) return hipErrorInvalidValue;
  return stream_launch(count, lins, K, X, M, r, s, part, tpart, counters, T, st);
}

}  // namespace qlora
