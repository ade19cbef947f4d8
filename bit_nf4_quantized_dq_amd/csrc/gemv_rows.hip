// Weight-streaming forward for few tokens (M <= 4) on weights of at least 4096 rows and a
// reduction of 2048 or 4096: Y = X w_hat^T + s (X A^T) B^T in one launch, one workgroup per
// 16 weight rows over the whole reduction.
//
// At small batch the layer is bound by reading the 4-bit weights ("QLoRA -- Fine-Tuning a 65B
// Model on One GPU", "Pitfalls": small-batch generation is memory-bound, and 4 bits leave less
// to read); each weight is decoded on chip from its code ("QLoRA: Quantize Base Weights to
// 4-Bit", Section 3).  With whole rows per workgroup no partial sums cross workgroups, and
// each wavefront works through its blocks in the order their loads were issued, so the
// decode and MFMA of a block start as soon as that block has landed.
//
// Work split.  Wavefront w takes blocks [w NBW, (w + 1) NBW) of the workgroup's 16 rows.  It
// loads its slice of X (M loads of 16 bytes per lane, one activation row each), then per
// block 8 bytes of codes per lane (the lane's row n = lane % 16, code words 2g and 2g + 1 of
// the block, g = lane / 16), after the 8-bit constants of its row's blocks.  While the codes
// travel, the workgroup builds in LDS a byte-pair table (for each code byte, the BF16 levels
// of its two nibbles, one copy per lane so that 64 lookups hit 64 banks) and the X slices.  A
// code byte holds weights e_i and e_{i+4} of its 8-weight run, so one v_perm (the address) and
// one LDS read give the pair (e_i, e_{i+4}); X is parked in the same order (x0 x4 x1 x5 x2 x6
// x3 x7 per 8), which leaves each product unchanged.  Barriers wait for LDS accesses only, so
// the codes stay in flight across them.  Two MFMA 16x16x32 steps cover a block, all 32 reduction indices of a step inside
// that block, so the block constant scales the 16x16 partial product once before it joins the
// accumulator.  Tokens past M read row M - 1, whose products land in output rows that are
// never written.  The eight wavefronts' sums meet in LDS in a fixed order.
//
// Adapter.  T = X A^T needs the whole reduction, so workgroup j < r forms column j of T first:
// each wavefront takes the dot product of its X slices with its slice of row j of A in
// registers (8 products per lane, then a fixed-order sum across the lanes) and parks it in LDS
// before the barrier that publishes the X slices, so T[m][j] is complete right after that
// barrier, while the codes are still in flight.  The workgroup then writes bf16(s T[m][j])
// with a tag into a private block of words of every workgroup, in the workspace head.  Each
// workgroup, after its rows, reads its M x r words until all carry the tag, applies (s T) B^T
// for its rows on MFMA, writes Y and then clears the words.  Each word block is read and cleared by its one owner, so the head is zero again
// after every call and a stale T is never taken for a new one, with no counter shared between
// workgroups.  Workgroups 0 .. r-1 are dispatched first and write T before they wait on
// anything, so no reader waits on a workgroup that has not started.
#include "qlora_device.h"
#include "qlora_host.h"

namespace qlora {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kRows = 16;            // weight rows per workgroup
constexpr int kMaxM = 4;             // tokens per call on this path
constexpr uint32_t kTag = 0x10000u;  // marks a written word (tag | bf16 bits)
constexpr size_t kHeadUse = QLORA_WS_COUNTER_BYTES;

struct RowsArgs {
  const uint8_t* codes;
  const uint8_t* code8;
  const float* c2s;
  const float* mu;
  int64_t N, K;
  const uint16_t* X;
  const uint16_t* A;
  const uint16_t* B;
  uint16_t* Y;
  uint16_t* T_save;
  uint32_t* words;  // [workgroups][M][r] (tag | bf16(s T)), zero between calls
  int32_t M, r;
  float s;
};

// LDS.  The byte-pair table comes first, at address 0, so a lookup address is the v_perm
// result itself: entry (byte v, lane l) at 256 v + 4 l.
template <int NBW>
struct RowsLds {
  uint32_t pair[256 * 64];
  uint4 x[kWaves][kMaxM][8 * NBW];  // X rows 0..M-1 of the slice
  f32x4_t red[kWaves][64];
  float tp[kWaves][kMaxM];  // per wavefront: its slice's part of T[m][c] (workgroup c < r)
};

// Workgroup barrier that waits for this wavefront's LDS accesses only, so global loads in
// flight (the codes) stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("s_barrier" ::: "memory");
}

__device__ __forceinline__ uint32_t byte_of(uint2 w, int i) {
  return ((i < 4 ? w.x : w.y) >> (8 * (i & 3))) & 0xFFu;
}

// 8 BF16 values x0..x7 (4 dwords) reordered to x0 x4 x1 x5 x2 x6 x3 x7.
__device__ __forceinline__ uint4 nibble_order(uint4 v) {
  return make_uint4(__builtin_amdgcn_perm(v.z, v.x, 0x05040100u), __builtin_amdgcn_perm(v.z, v.x, 0x07060302u),
                    __builtin_amdgcn_perm(v.w, v.y, 0x05040100u), __builtin_amdgcn_perm(v.w, v.y, 0x07060302u));
}

// BF16 bits of the levels named by the four index bytes of idx (values 0..15), one per
// 16-bit half: lo = levels of bytes 0, 1; hi = levels of bytes 2, 3.
__device__ __forceinline__ void levels4(const Lut& L, uint32_t idx, uint32_t& lo, uint32_t& hi) {
  const uint32_t idx8 = idx ^ 0x08080808u;
  const uint32_t m = nib_mask(idx);
  const uint32_t bl = lut16(idx, idx8, m, L.lo[0], L.lo[1], L.lo[2], L.lo[3]);  // low bytes
  const uint32_t bh = lut16(idx, idx8, m, L.hi[0], L.hi[1], L.hi[2], L.hi[3]);  // high bytes
  lo = __builtin_amdgcn_perm(bh, bl, 0x05010400u);
  hi = __builtin_amdgcn_perm(bh, bl, 0x07030602u);
}

// Wavefront w writes entries v = 32 w .. 32 w + 31 of the byte-pair table (8 KB): store q of
// lane l fills the 16 bytes at offset 16 (64 q + l) of that range, i.e. copies 4 (l % 16) ..
// +3 of entry v = 32 w + 4 q + l / 16, so consecutive lanes write consecutive bytes.  The
// entry's high nibble, 2 w + q / 4, is the same for the whole wavefront; its low nibble is
// 4 (q % 4) + l / 16.
__device__ __forceinline__ void build_pairs(const Lut& L, uint32_t* pair, int wave, int lane) {
  const uint32_t g = (uint32_t)lane >> 4;
  uint32_t lo01, lo23;  // levels of low nibbles g, 4 + g, 8 + g, 12 + g
  levels4(L, 0x0C080400u + g * 0x01010101u, lo01, lo23);
  uint32_t hi01, unused;  // levels of high nibbles 2 w, 2 w + 1
  levels4(L, (uint32_t)(2 * wave) * 0x0101u + 0x0100u, hi01, unused);
  (void)unused;
  const uint32_t lo[4] = {lo01 & 0xFFFFu, lo01 >> 16, lo23 & 0xFFFFu, lo23 >> 16};
  const uint32_t hi[2] = {hi01 << 16, hi01 & 0xFFFF0000u};
  uint4* dst = reinterpret_cast<uint4*>(pair + 32 * 64 * wave) + lane;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const uint32_t e = lo[q & 3] | hi[q >> 2];
    dst[64 * q] = make_uint4(e, e, e, e);
  }
}

// The 8 weights of one code word (element order e0 e4 e1 e5 e2 e6 e3 e7) as an MFMA operand:
// per byte, v_perm forms the table address (byte << 8 | 4 lane) and one LDS read returns the
// pair.
__device__ __forceinline__ bf16x8_t lookup8(const uint32_t* pair, uint32_t u, uint32_t lane4) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t addr = __builtin_amdgcn_perm(u, lane4, 0x0C0C0000u | ((4u + i) << 8));
    w[i] = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(pair) + addr);
  }
  return as_bf16x8(w);
}

// The operands the loads need come first, as scalars: the leading argument dwords (14 here)
// are preloaded into SGPRs (a by-value struct would not be), so the loads issue without
// waiting for the argument block.  mu (loaded after the codes) and the rest follow.
struct RowsRest {
  const uint16_t* B;
  uint16_t* Y;
  uint16_t* T_save;
  uint32_t* words;
  float s;
};

template <int NBW>  // blocks of 64 weights per wavefront: K = 64 * 8 * NBW
__global__ __launch_bounds__(kThreads) void k_gemv_rows(const uint16_t* X, const uint16_t* A, const uint8_t* code8,
                                                        const float* c2s, const uint8_t* codes, int32_t N32,
                                                        int32_t K32, int32_t M32, int32_t r32, const float* mu_p,
                                                        RowsRest rest, Lut L) {
  RowsArgs a;
  a.codes = codes;
  a.code8 = code8;
  a.c2s = c2s;
  a.mu = mu_p;
  a.N = N32;
  a.K = K32;
  a.X = X;
  a.A = A;
  a.B = rest.B;
  a.Y = rest.Y;
  a.T_save = rest.T_save;
  a.words = rest.words;
  a.M = M32;
  a.r = r32;
  a.s = rest.s;
  __shared__ RowsLds<NBW> S;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int64_t K = a.K, N = a.N;
  const int M = a.M, r = a.r;
  const int c = (int)blockIdx.x;
  const bool producer = c < r;  // forms column c of T first
  constexpr int kNb = 8 * NBW;  // blocks per row
  const int64_t row0 = (int64_t)c * kRows;
  const int64_t n = row0 + l16;  // this lane's weight row
  const int b0 = wave * NBW;     // first block of this wavefront
  const int64_t k0 = (int64_t)b0 * 64;

  // ---- loads in the order of use: X and A slices, block constants, codes
  const rsrc_t rx = make_rsrc(a.X, (int64_t)M * K * 2);
  uint4 xv[kMaxM + 1];
#pragma unroll
  for (int m = 0; m < kMaxM; ++m)
    xv[m] = bload16(rx, (m < M && lane < 8 * NBW) ? (uint32_t)((m * K + k0 + 8 * lane) * 2) : kOOB);
  {
    const rsrc_t ra = make_rsrc(a.A + (int64_t)c * K, K * 2);
    xv[kMaxM] = bload16(ra, (producer && lane < 8 * NBW) ? (uint32_t)((k0 + 8 * lane) * 2) : kOOB);
  }
  // the lane's row's block constants (8-bit codes of its NBW blocks, and the second-level
  // scales of the first and last of them: a row's run of blocks meets at most one group start)
  const int64_t blk0 = n * kNb + b0;
  const rsrc_t r8 = make_rsrc(a.code8, N * kNb);
  const rsrc_t r2 = make_rsrc(a.c2s, ((N * kNb + 255) / 256) * 4);
  uint2 c8w;
  if (NBW == 8) c8w = bload8(r8, (uint32_t)blk0);
  else c8w = make_uint2(bload4(r8, (uint32_t)blk0), 0u);
  const float c2a = __uint_as_float(bload4(r2, (uint32_t)((blk0 >> 8) * 4)));
  const float c2b = __uint_as_float(bload4(r2, (uint32_t)(((blk0 + NBW - 1) >> 8) * 4)));
  const rsrc_t rc = make_rsrc(a.codes + row0 * (K / 2), kRows * (K / 2));
  uint2 cr[NBW];
#pragma unroll
  for (int b = 0; b < NBW; ++b) cr[b] = bload8(rc, (uint32_t)(l16 * (K / 2) + 32 * (b0 + b) + 8 * g));
  const float mu = __uint_as_float(bload4(make_rsrc(a.mu, 4), 0u));  // used with the codes

  // ---- while the codes travel: the byte-pair table, the X slices and this wavefront's part
  // of column c of T (zero outside the producers, whose A slice is read out of range)
  build_pairs(L, S.pair, wave, lane);
#pragma unroll
  for (int m = 0; m < kMaxM; ++m)
    if (m < M && lane < 8 * NBW) S.x[wave][m][lane] = nibble_order(xv[m]);
  {
    const uint32_t av[4] = {xv[kMaxM].x, xv[kMaxM].y, xv[kMaxM].z, xv[kMaxM].w};
#pragma unroll
    for (int m = 0; m < kMaxM; ++m) {
      const uint32_t xw[4] = {xv[m].x, xv[m].y, xv[m].z, xv[m].w};
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        d = fmaf(bf16lo_to_f32(xw[e]), bf16lo_to_f32(av[e]), d);
        d = fmaf(bf16hi_to_f32(xw[e]), bf16hi_to_f32(av[e]), d);
      }
      if (m < M) {  // uniform: every lane takes part in the sum
        const float t = wave_sum(d);
        if (lane == 0) S.tp[wave][m] = t;
      }
    }
  }
  lds_barrier();

  // every X operand of the wavefront's blocks into registers at once (one LDS wait)
  const int mx = l16 < M ? l16 : M - 1;  // X row of this lane's operand
  uint4 xo[NBW][2];
#pragma unroll
  for (int b = 0; b < NBW; ++b)
#pragma unroll
    for (int s = 0; s < 2; ++s) xo[b][s] = S.x[wave][mx][8 * b + 2 * g + s];
  const f32x4_t z = {0.f, 0.f, 0.f, 0.f};

  // ---- workgroup c < r: column c of T (the wavefronts' parts in a fixed order) into every
  // workgroup's words
  if (producer) {
    const int nwg = (int)gridDim.x;
    for (int i = tid; i < nwg * M; i += kThreads) {  // word (workgroup i / M, token i % M)
      const int m = i % M;
      float t = S.tp[0][m];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) t += S.tp[w][m];
      if (i < M && a.T_save) a.T_save[m * r + c] = (uint16_t)(pack_bf16x2(t, 0.f) & 0xFFFFu);
      const uint32_t w = kTag | (pack_bf16x2(a.s * t, 0.f) & 0xFFFFu);
      __hip_atomic_store(a.words + (int64_t)i * r + c, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
  }

  // ---- this wavefront's share of the rows' product, block by block as the codes land
  // the lookups of block b + 1 are issued before the MFMAs of block b
  const uint32_t lane4 = 4u * lane;
  f32x4_t acc = z;
  bf16x8_t w0 = lookup8(S.pair, cr[0].x, lane4), w1 = lookup8(S.pair, cr[0].y, lane4);
#pragma unroll
  for (int b = 0; b < NBW; ++b) {
    const bf16x8_t u0 = w0, u1 = w1;
    if (b + 1 < NBW) {
      w0 = lookup8(S.pair, cr[b + 1 < NBW ? b + 1 : b].x, lane4);
      w1 = lookup8(S.pair, cr[b + 1 < NBW ? b + 1 : b].y, lane4);
    }
    f32x4_t p = mfma16x16x32(as_bf16x8(xo[b][0]), u0, z);
    p = mfma16x16x32(as_bf16x8(xo[b][1]), u1, p);
    const float c2 = (((blk0 + b) >> 8) == (blk0 >> 8)) ? c2a : c2b;
    const float cb = block_scale(byte_of(c8w, b), c2, mu);
    acc[0] = fmaf(cb, p[0], acc[0]);
    acc[1] = fmaf(cb, p[1], acc[1]);
    acc[2] = fmaf(cb, p[2], acc[2]);
    acc[3] = fmaf(cb, p[3], acc[3]);
  }
  S.red[wave][lane] = acc;
  // wavefront 0 issues its first read of the T words (they were written long before, so the
  // read is usually the only one) and the B rows of the first rank step before the barrier,
  // so that both travel while the other wavefronts finish
  uint32_t* mine = a.words + (int64_t)c * M * r;
  const rsrc_t rb = make_rsrc(a.B, N * r * 2);
  uint32_t tw[8], e[8];  // e: B[n][8 g .. 8 g + 7], element loads (B carries no alignment promise)
  if (wave == 0) {
    const bool live0 = l16 < M && 8 * g < r;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      tw[i] = live0 ? __hip_atomic_load(mine + l16 * r + 8 * g + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) : kTag;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      e[i] = __builtin_amdgcn_raw_buffer_load_b16(rb, 8 * g < r ? (int)((n * r + 8 * g + i) * 2) : (int)kOOB, 0, 0);
  }
  lds_barrier();
  if (wave != 0) return;

  // ---- wavefront 0: fixed-order sum, adapter term, output (lane holds D[4 g + v][l16])
  f32x4_t y = S.red[0][lane];
  for (int w = 1; w < kWaves; ++w) {
    const f32x4_t v = S.red[w][lane];
    y[0] += v[0]; y[1] += v[1]; y[2] += v[2]; y[3] += v[3];
  }
  for (int q0 = 0; q0 < r; q0 += 32) {
    // A operand: bf16(s T[m][q0 + 8 g .. +7]) from this workgroup's words; B operand: B[n][same]
    const int j0 = q0 + 8 * g;
    const bool live = l16 < M && j0 < r;  // r % 8 == 0: a live lane's 8 ranks all exist
    if (q0) {  // later rank steps: B rows loaded here (the first step's came with its words)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        e[i] = __builtin_amdgcn_raw_buffer_load_b16(rb, j0 < r ? (int)((n * r + j0 + i) * 2) : (int)kOOB, 0, 0);
    }
    bool ready = false;
    // bounded wait (about 2^20 polls): should the words never arrive, the outputs become NaN
    // instead of the wavefront spinning forever.  The first step's first read was issued above.
    for (int it = 0; !ready && it < (1 << 20); ++it) {
      if (it || q0) {
        if (it) __builtin_amdgcn_s_sleep(2);
#pragma unroll
        for (int i = 0; i < 8; ++i)
          tw[i] = live ? __hip_atomic_load(mine + l16 * r + j0 + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) : kTag;
      }
      ready = true;
#pragma unroll
      for (int i = 0; i < 8; ++i) ready = ready && (tw[i] & 0xFFFF0000u) == kTag;
    }
    if (!ready) {
#pragma unroll
      for (int i = 0; i < 8; ++i) tw[i] = kTag | 0x7FC0u;
    }
    uint32_t tv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) tv[i] = live ? ((tw[2 * i] & 0xFFFFu) | (tw[2 * i + 1] << 16)) : 0u;
    const uint32_t bw[4] = {(e[0] & 0xFFFFu) | (e[1] << 16), (e[2] & 0xFFFFu) | (e[3] << 16),
                            (e[4] & 0xFFFFu) | (e[5] << 16), (e[6] & 0xFFFFu) | (e[7] << 16)};
    y = mfma16x16x32(as_bf16x8(tv), as_bf16x8(bw), y);
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int mm = 4 * g + v;
    if (mm < M) a.Y[mm * N + n] = (uint16_t)(pack_bf16x2(y[v], 0.f) & 0xFFFFu);
  }
  // the words read, cleared for the next call: after the stores of Y, which then wait for
  // nothing but the loads they use
  for (int q0 = 0; q0 < r; q0 += 32) {
    const int j0 = q0 + 8 * g;
    if (l16 < M && j0 < r) {
#pragma unroll
      for (int i = 0; i < 8; ++i) __hip_atomic_store(mine + l16 * r + j0 + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
  }
}

}  // namespace

bool gemv_rows_fits(int64_t N, int64_t K, int64_t M, int32_t r) {
  if (M < 1 || M > kMaxM || r < 1 || r > 128 || r % 8 != 0 || N % kRows != 0 || N / kRows < 256) return false;
  if (K != 2048 && K != 4096) return false;
  return N / kRows >= r && (size_t)(N / kRows) * M * r * 4 <= kHeadUse;  // the words fit the head
}

hipError_t launch_gemv_rows(const uint32_t* codes, const uint8_t* code8, const float* c2s, const float* mu,
                            int64_t N, int64_t K, const uint16_t* X, int64_t M, const uint16_t* A,
                            const uint16_t* B, int32_t r, float s, uint16_t* Y, uint16_t* T_save, void* head,
                            const Nf4Tables& T, hipStream_t st) {
  if (!gemv_rows_fits(N, K, M, r)) return hipErrorInvalidValue;
  RowsArgs a;
  a.codes = reinterpret_cast<const uint8_t*>(codes);
  a.code8 = code8;
  a.c2s = c2s;
  a.mu = mu;
  a.N = N;
  a.K = K;
  a.X = X;
  a.A = A;
  a.B = B;
  a.Y = Y;
  a.T_save = T_save;
  a.words = static_cast<uint32_t*>(head);
  a.M = (int32_t)M;
  a.r = r;
  a.s = s;
  Lut L;  // the unscaled level bytes only (a smaller argument block than the whole tables)
  for (int w = 0; w < 4; ++w) {
    L.lo[w] = T.lut_lo[w];
    L.hi[w] = T.lut_hi[w];
  }
  const dim3 grid((unsigned)(N / kRows));
  const RowsRest rest{a.B, a.Y, a.T_save, a.words, a.s};
  LaunchTimer t(3, st);
  if (K == 4096)
    hipExtLaunchKernelGGL(k_gemv_rows<8>, grid, dim3(kThreads), 0, st, t.start, t.stop, 0, a.X, a.A, a.code8, a.c2s,
                          a.codes, (int32_t)N, (int32_t)K, a.M, a.r, a.mu, rest, L);
  else
    hipExtLaunchKernelGGL(k_gemv_rows<4>, grid, dim3(kThreads), 0, st, t.start, t.stop, 0, a.X, a.A, a.code8, a.c2s,
                          a.codes, (int32_t)N, (int32_t)K, a.M, a.r, a.mu, rest, L);
  return hipGetLastError();
}

}  // namespace qlora
