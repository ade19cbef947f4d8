// Internal host-side declarations of the HIP library: the NF4 tables, kernel launchers
// (defined next to their kernels) and the launch-timing hook.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "qlora.h"
#include "qlora_tables.h"

namespace qlora {

void build_nf4_tables(Nf4Tables* t);
const Nf4Tables& nf4_tables();
// First-level codebooks: 0 NF4, 1 uniform INT4, 2 FP4 (E2M1 levels).
void build_codebook_tables(int codebook, Nf4Tables* t);
const Nf4Tables& codebook_tables(int codebook);

// sum over e = 1..255 of hist[e] * 2^(e - 150), computed exactly and rounded once to double
// (nearest, ties to even).  Bin e of the first quantize pass holds the integer sum of the
// significands (implicit bit included) of the block constants whose biased FP32 exponent is
// e; subnormal constants go to bin 1 with their fraction bits, which gives them the same
// weight 2^-149 per unit.
double exact_sum_to_double(const unsigned long long hist[256]);

// Start/stop events for one kernel launch when timing is enabled for its id (see
// qlora_timing_*), else null.  Launch with hipExtLaunchKernelGGL(..., t.start, t.stop, 0,
// ...): the runtime then stamps the kernel's own execution window into the events.
struct LaunchTimer {
  LaunchTimer(int kernel_id, hipStream_t s);
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};
// While one of these lives on a thread, launches made by that thread carry no timing events
// (creating them allocates): the entry point that allocates nothing holds one.
struct TimingOff {
  TimingOff();
  ~TimingOff();
};

// ---- the forward entry point in two steps (api.cpp): every argument check, then the
// launches on a workspace of at least fwd_workspace_bytes() whose counter head is zero.
int fwd_validate(const qlora_nf4dq_t* Wq, const uint16_t* X, int64_t M, const uint16_t* A, const uint16_t* B,
                 int32_t r, float alpha, const uint16_t* Y);
size_t fwd_workspace_bytes(int64_t M, int64_t d_out, int64_t d_in, int32_t r, int dq);
int fwd_enqueue(const qlora_nf4dq_t* Wq, const uint16_t* X, int64_t M, const uint16_t* A, const uint16_t* B,
                int32_t r, float alpha, uint16_t* Y, uint16_t* T_save, void* ws, hipStream_t stream);

// ---- quantize / dequantize (quantize.hip, dequant.hip)
// Pass 1 spreads its exponent sums over kHistCopies zeroed copies of the 256 bins (workgroup
// w adds into copy w % kHistCopies), then adds the copies into copy 0: hist holds
// kHistCopies * 256 counters.  One copy for all workgroups serialized thousands of 64-bit
// atomics on a few addresses (about 20 us per call).
constexpr int kHistCopies = 64;
hipError_t launch_quant_pass1(const void* W, bool w_bf16, uint32_t* codes, float* c1, unsigned long long* hist,
                              int* flag, int64_t n_words, const Nf4Tables& T, hipStream_t s);
hipError_t launch_quant_pass2(const float* c1, float mu, uint8_t* code8, float* c2s, float* mu_out,
                              int64_t n_blocks, int dq, hipStream_t s);
hipError_t launch_e4m3_encode(const float* in, uint8_t* out, int64_t n, hipStream_t s);
// dq: second-level format of the block constants (kDqE4M3 .. kDqNone; for kDqNone code8
// holds FP32 constants and c2s, mu are not read).
hipError_t launch_dequant(const uint32_t* codes, const uint8_t* code8, const float* c2s,
                          const float* mu, uint16_t* out, int64_t n_words, const Nf4Tables& T, int dq,
                          hipStream_t s);

// w_hat^T [K, N] BF16 (transposed decode; the dX operand).
hipError_t launch_dequant_t(const uint32_t* codes, const uint8_t* code8, const float* c2s,
                            const float* mu, int64_t N, int64_t K, uint16_t* out, const Nf4Tables& T, int dq,
                            hipStream_t s);

// ---- merged export (merge.hip): out [N, K] BF16 = bf16(w_hat + s B A), B [N, r], A [r, K]
hipError_t launch_merge(const uint32_t* codes, const uint8_t* code8, const float* c2s, const float* mu,
                        const uint16_t* A, const uint16_t* B, int64_t N, int64_t K, int32_t r, float s,
                        uint16_t* out, const Nf4Tables& T, int dq, hipStream_t st);

// ---- adapter optimizer step (adamw.hip): scalars formed on the host in FP64, rounded once
struct AdamWScalars {
  float decay;         // 1 - lr * weight_decay
  float b1, omb1;      // beta1, 1 - beta1
  float b2, omb2;      // beta2, 1 - beta2
  float step_size;     // lr / (1 - beta1^t)
  float inv_bc2_sqrt;  // 1 / sqrt(1 - beta2^t)
  float eps;
};
hipError_t launch_adamw(float* master, float* m, float* v, const uint16_t* grad, uint16_t* param, int64_t n,
                        const AdamWScalars& a, hipStream_t s);

// ---- LoRA skinny kernels (lora.hip)
// out[m][j] = sum_k P[m][k] Q(j, k) for j < R, Q [R, Kd] (q_transposed = 0) or [Kd, R] (1);
// out_s = bf16(scale * sum), out_u = bf16(sum), BF16 [M, R], either may be null.
hipError_t launch_lora_down(const uint16_t* P, const uint16_t* Q, int q_transposed, int64_t M, int32_t R, int64_t Kd,
                            float scale, uint16_t* out_s, uint16_t* out_u, hipStream_t s);
// out(j, c) = bf16(scale * sum_m U[m][j] V[m][c]); U [M, R], V [M, C]; out [R, C], or
// [C, R] when transposed.  part: FP32 [lora_grad_msplit(M, C)][R][C] scratch; counters: one
// arrival counter per 64-column tile, zero before the call and left zero after it.
int32_t lora_grad_msplit(int64_t M, int64_t C);
hipError_t launch_lora_grad(const uint16_t* U, const uint16_t* V, int64_t M, int32_t R, int64_t C, float scale,
                            int transposed, float* part, unsigned int* counters, uint16_t* out, hipStream_t s);
// The step's prologues as one launch each (E4M3 constants): the down-projection T = X A^T
// (t_s = scale T, t_u = T) with the decoded copy w_out = w_hat [N, K]; and G = dY B (g_s, g_u)
// with the transposed decoded copy wt_out = w_hat^T [K, N].
hipError_t launch_fwd_prologue(const uint16_t* X, const uint16_t* A, int64_t M, int32_t R, int64_t K, float scale,
                               uint16_t* t_s, uint16_t* t_u, const uint32_t* codes, const uint8_t* code8,
                               const float* c2s, const float* mu, int64_t N, uint16_t* w_out, const Nf4Tables& T,
                               hipStream_t s);
hipError_t launch_bwd_prologue(const uint16_t* dY, const uint16_t* B, int64_t M, int32_t R, int64_t N, float scale,
                               uint16_t* g_s, uint16_t* g_u, const uint32_t* codes, const uint8_t* code8,
                               const float* c2s, const float* mu, int64_t K, uint16_t* wt_out, const Nf4Tables& T,
                               hipStream_t s);
// Two such products in one launch (each with its own partials and counters), e.g. dA and dB
// of one backward.
hipError_t launch_lora_grad2(const uint16_t* U0, const uint16_t* V0, int64_t C0, int transposed0, float* part0,
                             unsigned int* counters0, uint16_t* out0, const uint16_t* U1, const uint16_t* V1,
                             int64_t C1, int transposed1, float* part1, unsigned int* counters1, uint16_t* out1,
                             int64_t M, int32_t R, float scale, hipStream_t s);

// ---- weight-streaming forward, M <= 16 (gemv.hip): one launch, split-K with FP32
// partials part [ksplit][M][N] and tpart [ksplit][M][r] in the workspace, and one arrival
// counter per row group (gemv_groups), zero before the call and left zero after it.
int32_t gemv_ksplit(int64_t N, int64_t K);
int64_t gemv_groups(int64_t N);
hipError_t launch_gemv_fwd(const uint32_t* codes, const uint8_t* code8, const float* c2s,
                           const float* mu, int64_t N, int64_t K, const uint16_t* X, int64_t M,
                           const uint16_t* A, const uint16_t* B, int32_t r, float s, uint16_t* Y,
                           uint16_t* T_save, float* part, float* tpart, unsigned int* counters,
                           const Nf4Tables& T, hipStream_t st);
// The same forward with whole rows per workgroup (gemv_rows.hip): used when gemv_rows_fits()
// and the large-weight stream below does not apply.  Its only workspace is the counter head
// (`head`, QLORA_WS_COUNTER_BYTES, zero before the call and left zero).
bool gemv_rows_fits(int64_t N, int64_t K, int64_t M, int32_t r);
hipError_t launch_gemv_rows(const uint32_t* codes, const uint8_t* code8, const float* c2s, const float* mu,
                            int64_t N, int64_t K, const uint16_t* X, int64_t M, const uint16_t* A,
                            const uint16_t* B, int32_t r, float s, uint16_t* Y, uint16_t* T_save, void* head,
                            const Nf4Tables& T, hipStream_t st);
// The same forward for large weights (gemv_stream.hip): used when gemv_stream_fits(); its
// reduction split comes from gemv_stream_plan() (same partial layout as above).
struct GemvPlan {
  int64_t groups;
  int32_t ksplit, nbs, nchunk, xpitch;
};
GemvPlan gemv_stream_plan(int64_t N, int64_t K, int64_t M, int32_t r);
bool gemv_stream_fits(int64_t N, int64_t K, int64_t M, int32_t r);
hipError_t launch_gemv_stream(const uint32_t* codes, const uint8_t* code8, const float* c2s,
                              const float* mu, int64_t N, int64_t K, const uint16_t* X, int64_t M,
                              const uint16_t* A, const uint16_t* B, int32_t r, float s, uint16_t* Y,
                              uint16_t* T_save, float* part, float* tpart, unsigned int* counters,
                              const Nf4Tables& T, hipStream_t st);
// Grouped form: count (2..4) linears that read the same X [M, K], each d_out a multiple of
// 256, run as one launch.  Partials: part [ksplit][M][sum of d_out], tpart [count][ksplit][M][r],
// with ksplit = gemv_stream_plan(sum of d_out, K, M, r).ksplit, and one arrival counter per
// row group of the launch (gemv_stream_plan(...).groups).
struct StreamLinear {
  const uint32_t* codes;
  const uint8_t* code8;
  const float* c2s;
  const float* mu;
  int64_t N;
  const uint16_t* A;
  const uint16_t* B;
  uint16_t* Y;
  uint16_t* T_save;
};
constexpr int kStreamMaxGroup = 4;
bool gemv_stream_group_fits(int count, const int64_t* N, int64_t K, int64_t M, int32_t r);
hipError_t launch_gemv_stream_group(int count, const StreamLinear* lins, int64_t K, const uint16_t* X, int64_t M,
                                    int32_t r, float s, float* part, float* tpart, unsigned int* counters,
                                    const Nf4Tables& T, hipStream_t st);

// ---- fused dequant MFMA GEMMs (gemm.hip)
// Y[M,N] = X[M,K] w_hat^T + L[M,r] B[N,r]^T, L = s*T (BF16, prescaled)
hipError_t launch_gemm_fwd(const uint32_t* codes, const uint8_t* code8, const float* c2s,
                           const float* mu, int64_t N, int64_t K, const uint16_t* X, int64_t M,
                           const uint16_t* L, const uint16_t* B, int32_t r, uint16_t* Y,
                           const Nf4Tables& T, hipStream_t st);
// dX[M,K] = dY[M,N] w_hat + Lg[M,r] A[r,K], Lg = s*G (BF16, prescaled)
hipError_t launch_gemm_dx(const uint32_t* codes, const uint8_t* code8, const float* c2s,
                          const float* mu, int64_t N, int64_t K, const uint16_t* dY, int64_t M,
                          const uint16_t* Lg, const uint16_t* A, int32_t r, uint16_t* dX,
                          const Nf4Tables& T, hipStream_t st);

// ---- BF16 GEMM over a decoded weight copy (gemm_nt.hip):
// C [M, F] = (A [F, Kr] B [M, Kr]^T)^T + L [M, r] Wl^T, Wl(f, j) at f*wl_fs + j*wl_js.
// With ksplit > 1 (gemm_nt_ksplit(): products of at most 128 tiles), the reduction is split
// over ksplit workgroups per tile; part is FP32 [ksplit][M][F] workspace and F % 16 == 0.
int32_t gemm_nt_ksplit(int64_t F, int64_t M, int64_t Kr);
hipError_t launch_gemm_nt(const uint16_t* A, int64_t F, const uint16_t* B, int64_t M, int64_t Kr,
                          const uint16_t* wl, int64_t wl_fs, int64_t wl_js, const uint16_t* L, int32_t r,
                          uint16_t* C, int kernel_id, hipStream_t st, float* part = nullptr, int32_t ksplit = 1);

// ---- element-wise steps of the MLP block (mlp.hip); n values, n % 8 == 0, 16-byte aligned
hipError_t launch_swiglu_fwd(const uint16_t* G, const uint16_t* U, uint16_t* H, int64_t n, hipStream_t st);
hipError_t launch_swiglu_bwd(const uint16_t* dH, const uint16_t* G, const uint16_t* U, uint16_t* dG, uint16_t* dU,
                             int64_t n, hipStream_t st);
hipError_t launch_add_bf16(const uint16_t* a, const uint16_t* b, uint16_t* c, int64_t n, hipStream_t st);
// n 32-bit zeros at p (the workspace's counter head)
hipError_t launch_zero_words(unsigned int* p, int64_t n, hipStream_t st);

}  // namespace qlora
