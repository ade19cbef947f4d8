// C ABI of the NF4 + double-quantized LoRA linear (declared in include/qlora.h).
// Validates arguments, carves the caller's workspace, picks launch shapes and enqueues the
// kernels.  The only host-side arithmetic of the method is the exact mean of the block
// constants for double quantization, folded from the per-exponent integer sums that the
// first quantize pass gathers.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <vector>

#include "qlora.h"
#include "qlora_host.h"

using namespace qlora;

namespace {

// Buffer descriptors address at most 4 GiB from their base: a 256-row operand tile of
// width d must stay below 2^32 bytes, and the codes of one weight below 2^31 bytes.
constexpr int64_t kMaxDim = int64_t(1) << 22;
constexpr int64_t kMaxElems = int64_t(1) << 32;

inline bool shape_ok(int64_t d_out, int64_t d_in) {
  return d_out >= 16 && d_in >= 64 && d_in % 64 == 0 && d_out % 16 == 0 && d_out <= kMaxDim && d_in <= kMaxDim &&
         d_out * d_in <= kMaxElems;
}

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int hip_status(hipError_t e) { return e == hipSuccess ? QLORA_OK : QLORA_ERR_HIP; }

int check_wq(const qlora_nf4dq_t* Wq) {
  if (!Wq || !Wq->codes || !Wq->code8) return QLORA_ERR_INVALID_ARG;
  if (Wq->block1 != 64 || Wq->block2 != 256) return QLORA_ERR_UNSUPPORTED;
  if (Wq->codebook < QLORA_CB_NF4 || Wq->codebook > QLORA_CB_FP4 || Wq->dq_format < QLORA_DQ_E4M3 ||
      Wq->dq_format > QLORA_DQ_NONE)
    return QLORA_ERR_UNSUPPORTED;
  if (Wq->dq_format != QLORA_DQ_NONE && (!Wq->c2s || !Wq->mu)) return QLORA_ERR_INVALID_ARG;
  if ((Wq->dq_format == QLORA_DQ_NONE) && (reinterpret_cast<uintptr_t>(Wq->code8) & 3u)) return QLORA_ERR_INVALID_ARG;
  if (!shape_ok(Wq->d_out, Wq->d_in)) return QLORA_ERR_BAD_SHAPE;
  if (!aligned16(Wq->codes)) return QLORA_ERR_INVALID_ARG;
  return QLORA_OK;
}

// The caller's workspace: present and large enough (WORKSPACE), 16-byte aligned (INVALID_ARG).
int check_ws(const void* ws, size_t ws_bytes, size_t need) {
  if (!ws || ws_bytes < need) return QLORA_ERR_WORKSPACE;
  return aligned16(ws) ? QLORA_OK : QLORA_ERR_INVALID_ARG;
}

int check_lora(int64_t M, int32_t r, float alpha) {
  // M < 2^24 keeps every [M, r] operand (r <= 128) below the 4 GiB reach of a buffer descriptor
  if (M < 1 || M >= (int64_t(1) << 24)) return QLORA_ERR_INVALID_ARG;
  if (r < 1 || r > 128) return QLORA_ERR_INVALID_ARG;
  if (!std::isfinite(alpha)) return QLORA_ERR_INVALID_ARG;
  return QLORA_OK;
}

// The first-level table of a weight's codebook.
inline const Nf4Tables& tables_of(const qlora_nf4dq_t* Wq) { return codebook_tables(Wq->codebook); }

// Only E4M3 constants are decoded inside the fused GEMV / GEMM kernels; the other formats
// decode once per call into a BF16 copy (k_dequant, k_dequant_t) at every token count.
inline bool decode_once(int64_t M, int dq);

constexpr int64_t kGemvMaxM = 16;
// From this many tokens on, the weight is decoded once into a BF16 copy in the workspace
// and multiplied by the plain BF16 GEMM; below it the fused kernels decode per tile.
constexpr int64_t kNtMinM = 1024;
inline bool decode_once(int64_t M, int dq) { return M >= kNtMinM || dq != QLORA_DQ_E4M3; }

// The M <= 16 forward: the large-weight stream when it applies, else whole rows per
// workgroup when the shape allows, else the split-reduction kernel.
inline bool rows_path(int64_t N, int64_t K, int64_t M, int32_t r) {
  return !gemv_stream_fits(N, K, M, r) && gemv_rows_fits(N, K, M, r);
}

// ---- workspace layouts
// Every workspace starts with the arrival counters of the split reductions: one 32-bit word
// per row group of an M <= 16 forward, or per 64-column tile of dA and of dB in a backward
// (dB's after dA's).  The head has one fixed size, so calls of any kind and shape can share a
// workspace without one call's partials landing on another's counters.  It must be zero
// before the first use; every call leaves it zero.
constexpr size_t kHead = QLORA_WS_COUNTER_BYTES;
constexpr int64_t kHeadWords = (int64_t)(kHead / sizeof(unsigned int));
inline unsigned int* head_counters(void* ws) { return static_cast<unsigned int*>(ws); }

struct FwdWs {
  size_t tpart, ypart, ls, wcopy, gpart, total;
  int32_t gsplit;  // reduction split of the decode-once GEMM (FP32 partials at gpart)
};
FwdWs fwd_ws(int64_t M, int64_t N, int64_t K, int32_t r, int dq) {
  FwdWs w{};
  size_t off = kHead;
  w.tpart = off;
  if (M <= kGemvMaxM && !decode_once(M, dq) && rows_path(N, K, M, r)) {
    w.ypart = w.ls = off;  // whole rows per workgroup: only the counter head
  } else if (M <= kGemvMaxM && !decode_once(M, dq)) {
    const int32_t ks = gemv_stream_fits(N, K, M, r) ? gemv_stream_plan(N, K, M, r).ksplit : gemv_ksplit(N, K);
    off = align_up(off + sizeof(float) * ks * M * r, 256);
    w.ypart = off;
    off = align_up(off + sizeof(float) * ks * M * N, 256);
    w.ls = off;
  } else {
    w.ypart = off;
    w.ls = off;
    off = align_up(off + 2 * M * r, 256);
    if (decode_once(M, dq)) {
      w.wcopy = off;
      off = align_up(off + 2 * (size_t)N * K, 256);
      w.gsplit = gemm_nt_ksplit(N, M, K);
      if (w.gsplit > 1) {
        w.gpart = off;
        off = align_up(off + sizeof(float) * (size_t)w.gsplit * M * N, 256);
      }
    }
  }
  w.total = std::max<size_t>(off, 256);
  return w;
}

struct BwdWs {
  size_t t, g, lg, cpa, cpb, wcopy, total;
};
BwdWs bwd_ws(int64_t M, int64_t N, int64_t K, int32_t r, int dq) {
  BwdWs w{};
  size_t off = kHead;
  w.t = off;
  off = align_up(off + 2 * M * r, 256);
  w.g = off;
  off = align_up(off + 2 * M * r, 256);
  w.lg = off;
  off = align_up(off + 2 * M * r, 256);
  w.cpa = off;  // dA and dB run concurrently: separate partials
  off = align_up(off + sizeof(float) * (int64_t)lora_grad_msplit(M, K) * r * K, 256);
  w.cpb = off;
  off = align_up(off + sizeof(float) * (int64_t)lora_grad_msplit(M, N) * r * N, 256);
  if (decode_once(M, dq)) {
    w.wcopy = off;
    off = align_up(off + 2 * (size_t)N * K, 256);
  }
  w.total = off;
  return w;
}

// Grouped forward (qlora_linear_fwd_multi): one weight-streaming launch over linears that
// share X, else one qlora_linear_fwd per linear in the same workspace.
struct GroupWs {
  bool one_launch;
  size_t tpart, ypart, total;
};
GroupWs group_ws(int count, const qlora_nf4dq_t* const* Wq, int64_t M, int32_t r) {
  GroupWs w{};
  int64_t N[kStreamMaxGroup];
  const int64_t K = Wq[0]->d_in;
  bool one = count >= 2 && M <= kGemvMaxM;
  for (int i = 0; i < count; ++i) {
    N[i] = Wq[i]->d_out;
    one = one && Wq[i]->dq_format == QLORA_DQ_E4M3 && Wq[i]->codebook == Wq[0]->codebook;
    w.total = std::max(w.total, fwd_ws(M, N[i], K, r, Wq[i]->dq_format).total);
  }
  w.one_launch = one && gemv_stream_group_fits(count, N, K, M, r);
  if (w.one_launch) {
    int64_t Nt = 0;
    for (int i = 0; i < count; ++i) Nt += N[i];
    const int32_t ks = gemv_stream_plan(Nt, K, M, r).ksplit;
    w.tpart = kHead;
    w.ypart = align_up(kHead + sizeof(float) * count * ks * M * r, 256);
    w.total = std::max(w.total, align_up(w.ypart + sizeof(float) * ks * M * Nt, 256));
  }
  return w;
}

int check_group(int count, const qlora_nf4dq_t* const* Wq) {
  if (count < 1 || count > kStreamMaxGroup || !Wq) return QLORA_ERR_INVALID_ARG;
  for (int i = 0; i < count; ++i) {
    int st = check_wq(Wq[i]);
    if (st) return st;
    if (Wq[i]->d_in != Wq[0]->d_in) return QLORA_ERR_BAD_SHAPE;
  }
  return QLORA_OK;
}

// MLP block (qlora_mlp_fwd / qlora_mlp_bwd): the BF16 activations of the block, then one
// region large enough for any of the block's linear calls.
struct MlpWs {
  size_t g, u, h, dh, dg, du, dxu, lin, lin_bytes, total;
};
int check_mlp(const qlora_nf4dq_t* Wg, const qlora_nf4dq_t* Wu, const qlora_nf4dq_t* Wd) {
  int st;
  if ((st = check_wq(Wg)) || (st = check_wq(Wu)) || (st = check_wq(Wd))) return st;
  if (Wg->d_in != Wu->d_in || Wg->d_out != Wu->d_out || Wd->d_out != Wg->d_in || Wd->d_in != Wg->d_out)
    return QLORA_ERR_BAD_SHAPE;
  return QLORA_OK;
}
// The three adapters of the MLP block (gate, up, down) and, for the backward, their gradient
// outputs: every pointer present and A (16-byte loads) aligned, checked before any launch.
int check_adapters(const uint16_t* const* A, const uint16_t* const* B, uint16_t* const* dA, uint16_t* const* dB) {
  for (int i = 0; i < 3; ++i) {
    if (!A[i] || !B[i] || !aligned16(A[i])) return QLORA_ERR_INVALID_ARG;
    if (dA && (!dA[i] || !dB[i])) return QLORA_ERR_INVALID_ARG;
  }
  return QLORA_OK;
}
MlpWs mlp_ws(bool bwd, int64_t M, const qlora_nf4dq_t* Wg, const qlora_nf4dq_t* Wu, const qlora_nf4dq_t* Wd,
             int32_t r) {
  MlpWs w{};
  const int64_t d = Wg->d_in, f = Wg->d_out;
  const size_t act = align_up(2 * (size_t)M * f, 256);
  // the linear calls' region comes first, so their counter head is the block's own head
  const qlora_nf4dq_t* gu[2] = {Wg, Wu};
  size_t lin = std::max(group_ws(2, gu, M, r).total, fwd_ws(M, d, f, r, Wd->dq_format).total);
  if (bwd) {
    lin = std::max({lin, bwd_ws(M, f, d, r, Wg->dq_format).total, bwd_ws(M, f, d, r, Wu->dq_format).total,
                    bwd_ws(M, d, f, r, Wd->dq_format).total});
  }
  w.lin = 0;
  w.lin_bytes = align_up(lin, 256);
  size_t off = w.lin_bytes;
  w.g = off;
  off += act;
  w.u = off;
  off += act;
  w.h = off;
  off += act;
  if (bwd) {
    w.dh = off;
    off += act;
    w.dg = off;
    off += act;
    w.du = off;
    off += act;
    w.dxu = off;
    off += align_up(2 * (size_t)M * d, 256);
  }
  w.total = off;
  return w;
}

// The quantize workspace keeps the counter head untouched too, so one buffer can serve
// every entry point.
size_t quant_ws(int64_t d_out, int64_t d_in) {
  const int64_t nb = d_out * d_in / 64;
  return kHead + align_up(sizeof(float) * nb, 256) + kHistCopies * 256 * sizeof(unsigned long long) + 256;
}

// ---- kernel timing
struct TimingState {
  std::mutex mu;
  unsigned mask = 0;  // bit i: kernel id i is timed
  std::vector<std::pair<hipEvent_t, hipEvent_t>> ev[QLORA_K_COUNT];
  size_t used[QLORA_K_COUNT] = {0};
};
TimingState& timing() {
  static TimingState t;
  return t;
}

}  // namespace

namespace qlora {

// ---- exact mean: value = sum_e S_e * 2^(e-150) (e >= 1), folded in a big integer and
// rounded once to double (nearest, ties to even).
double exact_sum_to_double(const unsigned long long hist[256]) {
  // bit i of the integer has weight 2^(i - 149); bin e contributes S_e << (e - 1)
  constexpr int kWords = 12;  // 384 bits > 253 + 64 + margin
  uint64_t big[kWords] = {0};
  for (int e = 1; e < 256; ++e) {
    const uint64_t s = hist[e];
    if (!s) continue;
    const int sh = e - 1, w = sh / 64, b = sh % 64;
    unsigned __int128 add = (unsigned __int128)s << b;
    for (int i = w; i < kWords && add; ++i) {
      const unsigned __int128 cur = (unsigned __int128)big[i] + (uint64_t)add;
      big[i] = (uint64_t)cur;
      add = (add >> 64) + (cur >> 64);
    }
  }
  int top = -1;
  for (int i = kWords - 1; i >= 0 && top < 0; --i)
    if (big[i]) top = i * 64 + 63 - __builtin_clzll(big[i]);
  if (top < 0) return 0.0;
  auto bit = [&](int i) -> uint64_t { return i < 0 ? 0 : (big[i / 64] >> (i % 64)) & 1u; };
  if (top < 53) {
    uint64_t v = 0;
    for (int i = top; i >= 0; --i) v = (v << 1) | bit(i);
    return std::ldexp((double)v, -149);
  }
  uint64_t mant = 0;
  for (int i = top; i > top - 53; --i) mant = (mant << 1) | bit(i);
  const int lsb_pos = top - 52;
  const uint64_t guard = bit(lsb_pos - 1);
  bool sticky = false;
  for (int i = lsb_pos - 2; i >= 0 && !sticky; --i) sticky = bit(i) != 0;
  if (guard && (sticky || (mant & 1))) mant += 1;  // may carry to 2^53: still exact in double
  return std::ldexp((double)mant, lsb_pos - 149);
}

namespace {
thread_local int t_timing_off = 0;
}  // namespace

TimingOff::TimingOff() { ++t_timing_off; }
TimingOff::~TimingOff() { --t_timing_off; }

LaunchTimer::LaunchTimer(int kernel_id, hipStream_t) {
  if (t_timing_off) return;
  TimingState& T = timing();
  std::lock_guard<std::mutex> lk(T.mu);
  if (kernel_id < 0 || kernel_id >= QLORA_K_COUNT || !((T.mask >> kernel_id) & 1)) return;
  auto& v = T.ev[kernel_id];
  if (T.used[kernel_id] == v.size()) {
    // timing-only events: no system-scope fence (an L2 write-back and invalidate) when they
    // are recorded, so they neither stall the stream nor cool the caches of the next launch
    hipEvent_t a, b;
    if (hipEventCreateWithFlags(&a, hipEventDisableSystemFence) != hipSuccess) return;
    if (hipEventCreateWithFlags(&b, hipEventDisableSystemFence) != hipSuccess) {
      (void)hipEventDestroy(a);
      return;
    }
    v.emplace_back(a, b);
  }
  const size_t idx = T.used[kernel_id]++;
  start = v[idx].first;
  stop = v[idx].second;
}

}  // namespace qlora

namespace qlora {

int fwd_validate(const qlora_nf4dq_t* Wq, const uint16_t* X, int64_t M, const uint16_t* A, const uint16_t* B,
                 int32_t r, float alpha, const uint16_t* Y) {
  int st = check_wq(Wq);
  if (st) return st;
  if ((st = check_lora(M, r, alpha))) return st;
  if (!X || !A || !B || !Y || !aligned16(X) || !aligned16(A) || !aligned16(Y)) return QLORA_ERR_INVALID_ARG;
  if (M <= kGemvMaxM && !decode_once(M, Wq->dq_format)) {
    const int64_t N = Wq->d_out, K = Wq->d_in;
    // one arrival counter per row group of the launch, in the workspace head
    if ((gemv_stream_fits(N, K, M, r) ? gemv_stream_plan(N, K, M, r).groups : gemv_groups(N)) > kHeadWords)
      return QLORA_ERR_BAD_SHAPE;
  }
  return QLORA_OK;
}

size_t fwd_workspace_bytes(int64_t M, int64_t d_out, int64_t d_in, int32_t r, int dq) {
  return fwd_ws(M, d_out, d_in, r, dq).total;
}

int fwd_enqueue(const qlora_nf4dq_t* Wq, const uint16_t* X, int64_t M, const uint16_t* A, const uint16_t* B,
                int32_t r, float alpha, uint16_t* Y, uint16_t* T_save, void* ws, hipStream_t stream) {
  const int64_t N = Wq->d_out, K = Wq->d_in;
  const int dq = Wq->dq_format;
  const FwdWs L = fwd_ws(M, N, K, r, dq);
  char* base = static_cast<char*>(ws);
  const float s = alpha / (float)r;
  const uint32_t* codes = reinterpret_cast<const uint32_t*>(Wq->codes);
  float* tpart = reinterpret_cast<float*>(base + L.tpart);
  if (M <= kGemvMaxM && !decode_once(M, dq)) {
    float* ypart = reinterpret_cast<float*>(base + L.ypart);
    if (rows_path(N, K, M, r))
      return hip_status(launch_gemv_rows(codes, Wq->code8, Wq->c2s, Wq->mu, N, K, X, M, A, B, r, s, Y, T_save, ws,
                                         tables_of(Wq), stream));
    if (gemv_stream_fits(N, K, M, r))
      return hip_status(launch_gemv_stream(codes, Wq->code8, Wq->c2s, Wq->mu, N, K, X, M, A, B, r, s, Y, T_save,
                                           ypart, tpart, head_counters(ws), tables_of(Wq), stream));
    return hip_status(launch_gemv_fwd(codes, Wq->code8, Wq->c2s, Wq->mu, N, K, X, M, A, B, r, s, Y, T_save, ypart,
                                      tpart, head_counters(ws), tables_of(Wq), stream));
  }
  // T = X A^T: s T (BF16) feeds the adapter slices of the GEMM; T itself is saved if asked
  uint16_t* ls = reinterpret_cast<uint16_t*>(base + L.ls);
  hipError_t e;
  if (decode_once(M, dq)) {
    uint16_t* wcopy = reinterpret_cast<uint16_t*>(base + L.wcopy);
    if (dq == QLORA_DQ_E4M3) {  // T and the decoded copy in one launch
      if ((e = launch_fwd_prologue(X, A, M, r, K, s, ls, T_save, codes, Wq->code8, Wq->c2s, Wq->mu, N, wcopy,
                                   tables_of(Wq), stream)) != hipSuccess)
        return QLORA_ERR_HIP;
    } else {
      if ((e = launch_lora_down(X, A, 0, M, r, K, s, ls, T_save, stream)) != hipSuccess) return QLORA_ERR_HIP;
      if ((e = launch_dequant(codes, Wq->code8, Wq->c2s, Wq->mu, wcopy, N * K / 8, tables_of(Wq), dq, stream)) !=
          hipSuccess)
        return QLORA_ERR_HIP;
    }
    // Y = X w_hat^T + (s T) B^T: A = w_hat [N, K], Wl = B [N, r] (f*r + j)
    e = launch_gemm_nt(wcopy, N, X, M, K, B, r, 1, ls, r, Y, QLORA_K_GEMM_FWD, stream,
                       L.gsplit > 1 ? reinterpret_cast<float*>(base + L.gpart) : nullptr, L.gsplit > 1 ? L.gsplit : 1);
    return hip_status(e);
  }
  if ((e = launch_lora_down(X, A, 0, M, r, K, s, ls, T_save, stream)) != hipSuccess) return QLORA_ERR_HIP;
  e = launch_gemm_fwd(codes, Wq->code8, Wq->c2s, Wq->mu, N, K, X, M, ls, B, r, Y, tables_of(Wq), stream);
  return hip_status(e);
}

}  // namespace qlora

extern "C" {

const char* qlora_strerror(int status) {
  switch (status) {
    case QLORA_OK: return "ok";
    case QLORA_ERR_INVALID_ARG: return "invalid argument";
    case QLORA_ERR_BAD_SHAPE: return "bad shape (need d_in % 64 == 0, d_out % 16 == 0)";
    case QLORA_ERR_UNSUPPORTED: return "unsupported block sizes (need 64, 256), codebook or format";
    case QLORA_ERR_NONFINITE: return "non-finite weight";
    case QLORA_ERR_WORKSPACE: return "workspace too small";
    case QLORA_ERR_HIP: return "HIP runtime error";
    case QLORA_ERR_SCRATCH: return "needs more than the fixed scratch of the no-allocation forward";
    default: return "unknown status";
  }
}

int qlora_quant_sizes(int64_t d_out, int64_t d_in, size_t* codes_bytes, size_t* code8_bytes, size_t* c2s_bytes) {
  if (!codes_bytes || !code8_bytes || !c2s_bytes) return QLORA_ERR_INVALID_ARG;
  if (!shape_ok(d_out, d_in)) return QLORA_ERR_BAD_SHAPE;
  const int64_t n = d_out * d_in, nb = n / 64;
  *codes_bytes = (size_t)(n / 2);
  *code8_bytes = (size_t)nb;
  *c2s_bytes = sizeof(float) * (size_t)((nb + 255) / 256);
  return QLORA_OK;
}

int qlora_workspace_size(int op, int64_t M, int64_t d_out, int64_t d_in, int32_t r, size_t* ws_bytes) {
  return qlora_workspace_size_fmt(op, M, d_out, d_in, r, QLORA_DQ_E4M3, ws_bytes);
}

int qlora_workspace_size_fmt(int op, int64_t M, int64_t d_out, int64_t d_in, int32_t r, int dq_format,
                             size_t* ws_bytes) {
  if (!ws_bytes) return QLORA_ERR_INVALID_ARG;
  if (!shape_ok(d_out, d_in)) return QLORA_ERR_BAD_SHAPE;
  if (dq_format < QLORA_DQ_E4M3 || dq_format > QLORA_DQ_NONE) return QLORA_ERR_UNSUPPORTED;
  if (op == QLORA_OP_QUANTIZE) {
    *ws_bytes = quant_ws(d_out, d_in);
    return QLORA_OK;
  }
  int st = check_lora(M, r, 1.0f);
  if (st) return st;
  if (op == QLORA_OP_FWD) *ws_bytes = fwd_ws(M, d_out, d_in, r, dq_format).total;
  else if (op == QLORA_OP_BWD) *ws_bytes = bwd_ws(M, d_out, d_in, r, dq_format).total;
  else return QLORA_ERR_INVALID_ARG;
  return QLORA_OK;
}

int qlora_workspace_init(void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!ws || !aligned16(ws)) return QLORA_ERR_INVALID_ARG;
  if (ws_bytes < kHead) return QLORA_ERR_WORKSPACE;
  return hip_status(launch_zero_words(head_counters(ws), kHeadWords, stream));
}

int qlora_format_sizes(int64_t d_out, int64_t d_in, int dq_format, size_t* codes_bytes, size_t* code8_bytes,
                       size_t* c2s_bytes) {
  if (dq_format < QLORA_DQ_E4M3 || dq_format > QLORA_DQ_NONE) return QLORA_ERR_UNSUPPORTED;
  int st = qlora_quant_sizes(d_out, d_in, codes_bytes, code8_bytes, c2s_bytes);
  if (st || dq_format != QLORA_DQ_NONE) return st;
  *code8_bytes *= 4;  // one FP32 constant per block
  *c2s_bytes = 0;
  return QLORA_OK;
}

int qlora_codebook(int codebook, float out16[16]) {
  if (!out16 || codebook < QLORA_CB_NF4 || codebook > QLORA_CB_FP4) return QLORA_ERR_INVALID_ARG;
  std::memcpy(out16, codebook_tables(codebook).q, sizeof(float) * 16);
  return QLORA_OK;
}

int qlora_nf4_codebook(float out16[16]) {
  if (!out16) return QLORA_ERR_INVALID_ARG;
  std::memcpy(out16, nf4_tables().q, sizeof(float) * 16);
  return QLORA_OK;
}

}  // extern "C"

namespace {

// Both quantize entry points: W is FP32 or BF16 (widened exactly on load).
int quantize_impl(const void* W, bool w_bf16, const qlora_nf4dq_t* Wq, float* host_mu, void* ws, size_t ws_bytes,
                  hipStream_t stream) {
  int st = check_wq(Wq);
  if (st) return st;
  if (!W || !aligned16(W)) return QLORA_ERR_INVALID_ARG;
  const int64_t n = Wq->d_out * Wq->d_in, nb = n / 64;
  if ((st = check_ws(ws, ws_bytes, quant_ws(Wq->d_out, Wq->d_in)))) return st;
  char* base = static_cast<char*>(ws) + kHead;
  float* c1 = reinterpret_cast<float*>(base);
  auto* hist = reinterpret_cast<unsigned long long*>(base + align_up(sizeof(float) * nb, 256));
  int* flag = reinterpret_cast<int*>(hist + kHistCopies * 256);
  hipError_t e = hipMemsetAsync(hist, 0, kHistCopies * 256 * sizeof(unsigned long long) + 256, stream);
  if (e != hipSuccess) return QLORA_ERR_HIP;
  const bool no_dq = Wq->dq_format == QLORA_DQ_NONE;  // then c1 itself is the stored constant
  e = launch_quant_pass1(W, w_bf16, reinterpret_cast<uint32_t*>(Wq->codes), no_dq ? reinterpret_cast<float*>(Wq->code8) : c1,
                         hist, flag, n / 8, tables_of(Wq), stream);
  if (e != hipSuccess) return QLORA_ERR_HIP;
  unsigned long long h_hist[256];
  int h_flag = 0;
  if (hipMemcpyAsync(h_hist, hist, sizeof(h_hist), hipMemcpyDeviceToHost, stream) != hipSuccess) return QLORA_ERR_HIP;
  if (hipMemcpyAsync(&h_flag, flag, sizeof(int), hipMemcpyDeviceToHost, stream) != hipSuccess) return QLORA_ERR_HIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return QLORA_ERR_HIP;
  if (h_flag) return QLORA_ERR_NONFINITE;
  if (no_dq) {
    if (host_mu) *host_mu = 0.f;
    return QLORA_OK;
  }
  const double mean = exact_sum_to_double(h_hist) / (double)nb;
  const float mu = (float)mean;
  if (host_mu) *host_mu = mu;
  e = launch_quant_pass2(c1, mu, Wq->code8, Wq->c2s, Wq->mu, nb, Wq->dq_format, stream);
  return hip_status(e);
}

}  // namespace

extern "C" {

int qlora_quantize(const float* W, const qlora_nf4dq_t* Wq, float* host_mu, void* ws, size_t ws_bytes,
                   hipStream_t stream) {
  return quantize_impl(W, false, Wq, host_mu, ws, ws_bytes, stream);
}

int qlora_quantize_bf16(const uint16_t* W, const qlora_nf4dq_t* Wq, float* host_mu, void* ws, size_t ws_bytes,
                        hipStream_t stream) {
  return quantize_impl(W, true, Wq, host_mu, ws, ws_bytes, stream);
}

int qlora_dequantize(const qlora_nf4dq_t* Wq, uint16_t* W_bf16, hipStream_t stream) {
  int st = check_wq(Wq);
  if (st) return st;
  if (!W_bf16 || !aligned16(W_bf16)) return QLORA_ERR_INVALID_ARG;
  const int64_t n = Wq->d_out * Wq->d_in;
  return hip_status(launch_dequant(reinterpret_cast<const uint32_t*>(Wq->codes), Wq->code8, Wq->c2s, Wq->mu,
                                   W_bf16, n / 8, tables_of(Wq), Wq->dq_format, stream));
}

int qlora_merge(const qlora_nf4dq_t* Wq, const uint16_t* A, const uint16_t* B, int32_t r, float alpha,
                uint16_t* W_out, hipStream_t stream) {
  int st = check_wq(Wq);
  if (st) return st;
  if ((st = check_lora(1, r, alpha))) return st;
  if (!A || !B || !W_out || !aligned16(A) || !aligned16(W_out)) return QLORA_ERR_INVALID_ARG;
  if ((r & 7) == 0 && !aligned16(B)) return QLORA_ERR_INVALID_ARG;
  const int64_t N = Wq->d_out, K = Wq->d_in;
  if ((N + 127) / 128 > 65535) return QLORA_ERR_BAD_SHAPE;  // grid rows of 128 weights
  return hip_status(launch_merge(reinterpret_cast<const uint32_t*>(Wq->codes), Wq->code8, Wq->c2s, Wq->mu, A, B, N, K,
                                 r, alpha / (float)r, W_out, tables_of(Wq), Wq->dq_format, stream));
}

int qlora_linear_fwd(const qlora_nf4dq_t* Wq, const uint16_t* X, int64_t M, const uint16_t* A, const uint16_t* B,
                     int32_t r, float alpha, uint16_t* Y, uint16_t* T_save, void* ws, size_t ws_bytes,
                     hipStream_t stream) {
  int st = qlora::fwd_validate(Wq, X, M, A, B, r, alpha, Y);
  if (st) return st;
  if ((st = check_ws(ws, ws_bytes, fwd_ws(M, Wq->d_out, Wq->d_in, r, Wq->dq_format).total))) return st;
  return qlora::fwd_enqueue(Wq, X, M, A, B, r, alpha, Y, T_save, ws, stream);
}

int qlora_workspace_size_multi(int count, const qlora_nf4dq_t* const* Wq, int64_t M, int32_t r, size_t* ws_bytes) {
  if (!ws_bytes) return QLORA_ERR_INVALID_ARG;
  int st = check_group(count, Wq);
  if (st) return st;
  if ((st = check_lora(M, r, 1.0f))) return st;
  *ws_bytes = group_ws(count, Wq, M, r).total;
  return QLORA_OK;
}

int qlora_linear_fwd_multi(int count, const qlora_nf4dq_t* const* Wq, const uint16_t* X, int64_t M,
                           const uint16_t* const* A, const uint16_t* const* B, int32_t r, float alpha,
                           uint16_t* const* Y, uint16_t* const* T_save, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
  int st = check_group(count, Wq);
  if (st) return st;
  if ((st = check_lora(M, r, alpha))) return st;
  if (!X || !A || !B || !Y || !aligned16(X)) return QLORA_ERR_INVALID_ARG;
  for (int i = 0; i < count; ++i)
    if (!A[i] || !B[i] || !Y[i] || !aligned16(A[i]) || !aligned16(Y[i])) return QLORA_ERR_INVALID_ARG;
  const GroupWs L = group_ws(count, Wq, M, r);
  if ((st = check_ws(ws, ws_bytes, L.total))) return st;
  if (!L.one_launch) {
    for (int i = 0; i < count; ++i) {
      st = qlora_linear_fwd(Wq[i], X, M, A[i], B[i], r, alpha, Y[i], T_save ? T_save[i] : nullptr, ws, ws_bytes,
                            stream);
      if (st) return st;
    }
    return QLORA_OK;
  }
  StreamLinear lins[kStreamMaxGroup];
  for (int i = 0; i < count; ++i)
    lins[i] = StreamLinear{reinterpret_cast<const uint32_t*>(Wq[i]->codes), Wq[i]->code8, Wq[i]->c2s, Wq[i]->mu,
                           Wq[i]->d_out, A[i], B[i], Y[i], T_save ? T_save[i] : nullptr};
  char* base = static_cast<char*>(ws);
  return hip_status(launch_gemv_stream_group(count, lins, Wq[0]->d_in, X, M, r, alpha / (float)r,
                                             reinterpret_cast<float*>(base + L.ypart),
                                             reinterpret_cast<float*>(base + L.tpart), head_counters(ws),
                                             tables_of(Wq[0]), stream));
}

int qlora_mlp_workspace_size(int op, int64_t M, const qlora_nf4dq_t* Wg, const qlora_nf4dq_t* Wu,
                             const qlora_nf4dq_t* Wd, int32_t r, size_t* ws_bytes) {
  if (!ws_bytes || (op != QLORA_OP_FWD && op != QLORA_OP_BWD)) return QLORA_ERR_INVALID_ARG;
  int st = check_mlp(Wg, Wu, Wd);
  if (st || (st = check_lora(M, r, 1.0f))) return st;
  *ws_bytes = mlp_ws(op == QLORA_OP_BWD, M, Wg, Wu, Wd, r).total;
  return QLORA_OK;
}

int qlora_mlp_fwd(const qlora_nf4dq_t* Wg, const qlora_nf4dq_t* Wu, const qlora_nf4dq_t* Wd, const uint16_t* X,
                  int64_t M, const uint16_t* const* A, const uint16_t* const* B, int32_t r, float alpha, uint16_t* Y,
                  uint16_t* G_save, uint16_t* U_save, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_mlp(Wg, Wu, Wd);
  if (st || (st = check_lora(M, r, alpha))) return st;
  if (!X || !A || !B || !Y || !aligned16(X) || !aligned16(Y)) return QLORA_ERR_INVALID_ARG;
  if ((st = check_adapters(A, B, nullptr, nullptr))) return st;
  if ((G_save && !aligned16(G_save)) || (U_save && !aligned16(U_save))) return QLORA_ERR_INVALID_ARG;
  const MlpWs L = mlp_ws(false, M, Wg, Wu, Wd, r);
  if ((st = check_ws(ws, ws_bytes, L.total))) return st;
  char* base = static_cast<char*>(ws);
  uint16_t* G = G_save ? G_save : reinterpret_cast<uint16_t*>(base + L.g);
  uint16_t* U = U_save ? U_save : reinterpret_cast<uint16_t*>(base + L.u);
  uint16_t* H = reinterpret_cast<uint16_t*>(base + L.h);
  void* lin = base + L.lin;
  const qlora_nf4dq_t* gu[2] = {Wg, Wu};
  uint16_t* GU[2] = {G, U};
  // gate and up read the same X: one grouped call (one weight-streaming launch at M <= 16)
  if ((st = qlora_linear_fwd_multi(2, gu, X, M, A, B, r, alpha, GU, nullptr, lin, L.lin_bytes, stream))) return st;
  if (launch_swiglu_fwd(G, U, H, M * Wg->d_out, stream) != hipSuccess) return QLORA_ERR_HIP;
  return qlora_linear_fwd(Wd, H, M, A[2], B[2], r, alpha, Y, nullptr, lin, L.lin_bytes, stream);
}

int qlora_mlp_bwd(const qlora_nf4dq_t* Wg, const qlora_nf4dq_t* Wu, const qlora_nf4dq_t* Wd, const uint16_t* X,
                  const uint16_t* dY, int64_t M, const uint16_t* const* A, const uint16_t* const* B, int32_t r,
                  float alpha, const uint16_t* G_saved, const uint16_t* U_saved, uint16_t* dX, uint16_t* const* dA,
                  uint16_t* const* dB, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_mlp(Wg, Wu, Wd);
  if (st || (st = check_lora(M, r, alpha))) return st;
  if (!X || !dY || !A || !B || !dX || !dA || !dB) return QLORA_ERR_INVALID_ARG;
  if (!aligned16(X) || !aligned16(dY) || !aligned16(dX)) return QLORA_ERR_INVALID_ARG;
  if ((st = check_adapters(A, B, dA, dB))) return st;
  if ((G_saved == nullptr) != (U_saved == nullptr)) return QLORA_ERR_INVALID_ARG;
  if (G_saved && (!aligned16(G_saved) || !aligned16(U_saved))) return QLORA_ERR_INVALID_ARG;
  const MlpWs L = mlp_ws(true, M, Wg, Wu, Wd, r);
  if ((st = check_ws(ws, ws_bytes, L.total))) return st;
  char* base = static_cast<char*>(ws);
  const int64_t f = Wg->d_out, d = Wg->d_in;
  void* lin = base + L.lin;
  const uint16_t* G = G_saved;
  const uint16_t* U = U_saved;
  if (!G) {  // recompute the block's inner activations (gradient checkpointing)
    uint16_t* GU[2] = {reinterpret_cast<uint16_t*>(base + L.g), reinterpret_cast<uint16_t*>(base + L.u)};
    const qlora_nf4dq_t* gu[2] = {Wg, Wu};
    if ((st = qlora_linear_fwd_multi(2, gu, X, M, A, B, r, alpha, GU, nullptr, lin, L.lin_bytes, stream))) return st;
    G = GU[0];
    U = GU[1];
  }
  uint16_t* H = reinterpret_cast<uint16_t*>(base + L.h);
  uint16_t* dH = reinterpret_cast<uint16_t*>(base + L.dh);
  uint16_t* dG = reinterpret_cast<uint16_t*>(base + L.dg);
  uint16_t* dU = reinterpret_cast<uint16_t*>(base + L.du);
  uint16_t* dXu = reinterpret_cast<uint16_t*>(base + L.dxu);
  if (launch_swiglu_fwd(G, U, H, M * f, stream) != hipSuccess) return QLORA_ERR_HIP;
  if ((st = qlora_linear_bwd(Wd, H, dY, M, A[2], B[2], r, alpha, nullptr, dH, dA[2], dB[2], lin, L.lin_bytes, stream)))
    return st;
  if (launch_swiglu_bwd(dH, G, U, dG, dU, M * f, stream) != hipSuccess) return QLORA_ERR_HIP;
  if ((st = qlora_linear_bwd(Wg, X, dG, M, A[0], B[0], r, alpha, nullptr, dX, dA[0], dB[0], lin, L.lin_bytes, stream)))
    return st;
  if ((st = qlora_linear_bwd(Wu, X, dU, M, A[1], B[1], r, alpha, nullptr, dXu, dA[1], dB[1], lin, L.lin_bytes, stream)))
    return st;
  return hip_status(launch_add_bf16(dX, dXu, dX, M * d, stream));
}

int qlora_linear_bwd(const qlora_nf4dq_t* Wq, const uint16_t* X, const uint16_t* dY, int64_t M, const uint16_t* A,
                     const uint16_t* B, int32_t r, float alpha, const uint16_t* T_saved, uint16_t* dX, uint16_t* dA,
                     uint16_t* dB, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_wq(Wq);
  if (st) return st;
  if ((st = check_lora(M, r, alpha))) return st;
  if (!X || !dY || !A || !B || !dA || !dB) return QLORA_ERR_INVALID_ARG;
  if (!aligned16(X) || !aligned16(dY) || !aligned16(A) || (dX && !aligned16(dX))) return QLORA_ERR_INVALID_ARG;
  const int64_t N = Wq->d_out, K = Wq->d_in;
  const int dq = Wq->dq_format;
  const BwdWs L = bwd_ws(M, N, K, r, dq);
  if ((st = check_ws(ws, ws_bytes, L.total))) return st;
  char* base = static_cast<char*>(ws);
  const float s = alpha / (float)r;
  uint16_t* t = reinterpret_cast<uint16_t*>(base + L.t);
  uint16_t* g = reinterpret_cast<uint16_t*>(base + L.g);
  uint16_t* lg = reinterpret_cast<uint16_t*>(base + L.lg);
  float* cpa = reinterpret_cast<float*>(base + L.cpa);
  float* cpb = reinterpret_cast<float*>(base + L.cpb);
  const uint32_t* codes = reinterpret_cast<const uint32_t*>(Wq->codes);
  hipError_t e;
  const uint16_t* T = T_saved;
  if (!T) {  // recompute T = X A^T
    if ((e = launch_lora_down(X, A, 0, M, r, K, 1.0f, t, nullptr, stream)) != hipSuccess) return QLORA_ERR_HIP;
    T = t;
  }
  // G = dY B (B [N, r] is read as the transposed operand); s G and G in BF16.  dX = dY w_hat +
  // (s G) A; with the decoded copy, G and the transposed decode share one launch (E4M3).
  const bool fused = dX && decode_once(M, dq) && dq == QLORA_DQ_E4M3;
  uint16_t* wcopy = reinterpret_cast<uint16_t*>(base + L.wcopy);
  if (fused) {
    if ((e = launch_bwd_prologue(dY, B, M, r, N, s, lg, g, codes, Wq->code8, Wq->c2s, Wq->mu, K, wcopy, tables_of(Wq),
                                 stream)) != hipSuccess)
      return QLORA_ERR_HIP;
  } else if ((e = launch_lora_down(dY, B, 1, M, r, N, s, lg, g, stream)) != hipSuccess) {
    return QLORA_ERR_HIP;
  }
  if (dX && decode_once(M, dq)) {
    if (!fused &&
        (e = launch_dequant_t(codes, Wq->code8, Wq->c2s, Wq->mu, N, K, wcopy, tables_of(Wq), dq, stream)) != hipSuccess)
      return QLORA_ERR_HIP;
    // A = w_hat^T [K, N], Wl(f, j) = A[j][f]: read in place from A [r, K] (f*1 + j*K)
    if ((e = launch_gemm_nt(wcopy, K, dY, M, N, A, 1, K, lg, r, dX, QLORA_K_GEMM_DX, stream)) != hipSuccess)
      return QLORA_ERR_HIP;
  } else if (dX) {
    if ((e = launch_gemm_dx(codes, Wq->code8, Wq->c2s, Wq->mu, N, K, dY, M, lg, A, r, dX, tables_of(Wq), stream)) !=
        hipSuccess)
      return QLORA_ERR_HIP;
  }
  // dA = s G^T X [r, K] and dB = s dY^T T, stored [N, r], in one launch (own partials and
  // arrival counters each)
  // (counters: dA's column tiles, then dB's, in the workspace head)
  unsigned int* cnt_a = head_counters(ws);
  unsigned int* cnt_b = cnt_a + (K + 63) / 64;
  if ((e = launch_lora_grad2(g, X, K, 0, cpa, cnt_a, dA, T, dY, N, 1, cpb, cnt_b, dB, M, r, s, stream)) != hipSuccess)
    return QLORA_ERR_HIP;
  return QLORA_OK;
}

int qlora_adamw_step(float* master, float* m, float* v, const uint16_t* grad, uint16_t* param, int64_t n,
                     int64_t step, float lr, float beta1, float beta2, float eps, float weight_decay,
                     hipStream_t stream) {
  if (n < 0 || step < 1) return QLORA_ERR_INVALID_ARG;
  if (!(std::isfinite(lr) && lr >= 0.f && beta1 >= 0.f && beta1 < 1.f && beta2 >= 0.f && beta2 < 1.f &&
        std::isfinite(eps) && eps > 0.f && std::isfinite(weight_decay) && weight_decay >= 0.f))
    return QLORA_ERR_INVALID_ARG;
  if (n == 0) return QLORA_OK;
  if (!master || !m || !v || !grad) return QLORA_ERR_INVALID_ARG;
  if (!aligned16(master) || !aligned16(m) || !aligned16(v) || (reinterpret_cast<uintptr_t>(grad) & 7u) ||
      (param && (reinterpret_cast<uintptr_t>(param) & 7u)))
    return QLORA_ERR_INVALID_ARG;
  const double t = (double)step, b1 = beta1, b2 = beta2;
  AdamWScalars a;
  a.decay = (float)(1.0 - (double)lr * (double)weight_decay);
  a.b1 = beta1;
  a.omb1 = (float)(1.0 - b1);
  a.b2 = beta2;
  a.omb2 = (float)(1.0 - b2);
  a.step_size = (float)((double)lr / (1.0 - std::pow(b1, t)));
  a.inv_bc2_sqrt = (float)(1.0 / std::sqrt(1.0 - std::pow(b2, t)));
  a.eps = eps;
  return hip_status(launch_adamw(master, m, v, grad, param, n, a, stream));
}

int qlora_e4m3_encode(const float* in, uint8_t* out, int64_t n, hipStream_t stream) {
  if (!in || !out || n < 0) return QLORA_ERR_INVALID_ARG;
  if (n == 0) return QLORA_OK;
  return hip_status(launch_e4m3_encode(in, out, n, stream));
}

int qlora_timing_enable(int kernel_mask) {
  TimingState& T = timing();
  std::lock_guard<std::mutex> lk(T.mu);
  T.mask = (unsigned)kernel_mask & ((1u << QLORA_K_COUNT) - 1u);
  for (int i = 0; i < QLORA_K_COUNT; ++i)
    if ((T.mask >> i) & 1) T.used[i] = 0;
  return QLORA_OK;
}

int qlora_timing_read(int kernel_id, double* total_ms, int64_t* launches) {
  if (kernel_id < 0 || kernel_id >= QLORA_K_COUNT || !total_ms || !launches) return QLORA_ERR_INVALID_ARG;
  TimingState& T = timing();
  std::lock_guard<std::mutex> lk(T.mu);
  double sum = 0.0;
  const size_t n = T.used[kernel_id];
  for (size_t i = 0; i < n; ++i) {
    auto& p = T.ev[kernel_id][i];
    if (hipEventSynchronize(p.second) != hipSuccess) return QLORA_ERR_HIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, p.first, p.second) != hipSuccess) return QLORA_ERR_HIP;
    sum += ms;
  }
  T.used[kernel_id] = 0;
  *total_ms = sum;
  *launches = (int64_t)n;
  return QLORA_OK;
}

}  // extern "C"
