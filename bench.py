"""Benchmark of the NF4 + double-quantized LoRA linear on one MI355X.

A step is one training pass of the hot path over one batch: forward (LoRA down-projection
T = X A^T, decode of the weight to a BF16 copy, BF16 MFMA GEMM Y = X w_hat^T + s T B^T) and
backward (G = dY B, transposed decode w_hat^T, BF16 MFMA GEMM dX = dY w_hat + s G A,
dA = s G^T X, dB = s dY^T T) of the 4096x4096 linear at M = 4096 tokens, r = 16,
alpha = 32, inputs resident in HBM.  value = algorithmic TFLOP/s of that step
(4MNK + 6Mr(N+K) per step) over the timed steps.

Also reported in the same JSON line: the roofline of the dominant kernel (algorithmic
FLOPs per launch over its average duration from timing-only HIP events recorded on the
launch stream inside the timed region -- on the two GEMM launches of its last EVENT_STEPS
steps, since each recorded event adds command-processor time to its step), a per-kernel
breakdown from a separate fully instrumented pass, the M = 1 weight-stream rate of the
same linear (128 distinct quantized copies rotated so every call reads HBM), the quantize
rate, the merged-export rate (w_hat + s B A to BF16 over the same rotated copies), the
AdamW step over the 41.9M adapter parameters of a Llama-3-8B-shaped model, an error study of
the format variants (codebook x second-level format: bits/weight, reconstruction error,
decode time), the other two named workloads (all seven linears of a Llama-3-8B-shaped layer
at M = 8192, fwd + bwd; a 70B-class model's 560 linears, ~35 GB of NF4+DQ resident, forward at
M = 1 by graph replay, one launch per linear and with q/k/v and gate/up grouped, and at
M = 2048), the Llama-3-8B-shaped MLP block chained through its activation (fwd + bwd, with
saved or recomputed activations), and the CPU oracle timed on a bounded sample of the same
workload.

  python bench.py [--gpus 1] [--steps 100] [--warmup 100] [--no-cpu-baseline] [--no-extra]

The default warm-up (about 30 ms of steps) lets the clock under sustained MFMA load settle:
on a fresh box the first ~60 steps run up to 13% slower than the rest.
  python bench.py --pmc-pass    # 2 steps, one merge, one AdamW step, two M = 1 and two
                                # M = 16 calls on the step's weight, two M = 1 calls and one
                                # M = 2048 call on a 28672x8192 weight, one M = 2048 call on a
                                # 1024x8192 weight and a 256 MiB device copy (the counter
                                # calibration), for counter runs
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

METRIC = "NF4+DQ linear fwd+bwd TFLOP/s at M=4096; weight-stream GB/s at M=1"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0


# Counters per launch from four rocprofv3 passes of `bench.py --pmc-pass` (FETCH_SIZE;
# WRITE_SIZE; SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_MFMA, SQ_INSTS_VALU, SQ_INSTS_LDS and others;
# SQ_LDS_BANK_CONFLICT, SQ_INSTS_SALU and others).  HBM bytes are FETCH_SIZE scaled by 2.0 and
# WRITE_SIZE by 1.0, the factors that make a plain 256 MiB device copy read and write 256 MiB.
# SQ_* counts are summed over the whole chip.  A record holds only for the kernel source it
# was taken on: when that file's SHA-1 differs, its figures are reported as null.
COUNTERS = {
    "gemm_nt": {"source": "bit_nf4_quantized_dq_amd/csrc/gemm_nt.hip",
                "sha1": "5ce5dbfd0aa38821b99f12d226e7a0e43790f4b7",
                "read_bytes": 202_359_398, "write_bytes": 33_554_432,
                "mfma_insts": 4_243_456, "mfma_busy_cycles": 135_790_592, "valu_insts": 5_626_368,
                "lds_insts": 3_244_032, "lds_bank_conflict_cycles": 65_536, "salu_insts": 3_279_616},
    # the step's HBM-bound launches (4096 x 4096, M = 4096, r = 16)
    "fwd_prologue": {"source": "bit_nf4_quantized_dq_amd/csrc/lora.hip",
                     "sha1": "0b8df2d485634ad8f60dc2dba058b04007f6deeb",
                     "read_bytes": 43_486_144, "write_bytes": 33_816_576},
    "bwd_prologue": {"source": "bit_nf4_quantized_dq_amd/csrc/lora.hip",
                     "sha1": "0b8df2d485634ad8f60dc2dba058b04007f6deeb",
                     "read_bytes": 45_822_208, "write_bytes": 33_816_576},
    "lora_grad2": {"source": "bit_nf4_quantized_dq_amd/csrc/lora.hip",
                   "sha1": "0b8df2d485634ad8f60dc2dba058b04007f6deeb",
                   "read_bytes": 71_515_008, "write_bytes": 2_379_776},
    "merge": {"source": "bit_nf4_quantized_dq_amd/csrc/merge.hip",
              "sha1": "aa1649879396b227b61d065c057ec39a4962a28a",
              "read_bytes": 11_910_758, "write_bytes": 33_554_534},
    "adamw": {"source": "bit_nf4_quantized_dq_amd/csrc/adamw.hip",
              "sha1": "513130524f3da5219d61f8dcabd1c76bb0828e6f",
              "read_bytes": 587_329_946, "write_bytes": 587_202_560},
    # the 4096 x 4096 weight at M = 1 (whole-row stream) and at M = 16 (split-K stream)
    "gemv_rows_M1": {"source": "bit_nf4_quantized_dq_amd/csrc/gemv_rows.hip",
                     "sha1": "3933ee32978a1b227ae3a8eecc2239423da8f759",
                     "read_bytes": 9_203_392, "write_bytes": 270_336, "weights": 4096 * 4096,
                     "mfma_insts": 33_024, "valu_insts": 826_768, "lds_insts": 188_672, "lds_bank_conflict_cycles": 0},
    "gemv_fused_M16": {"source": "bit_nf4_quantized_dq_amd/csrc/gemv.hip",
                       "sha1": "722bc599e5742326b6648d9d31c04341b0eaa8f2",
                       "read_bytes": 13_233_664, "write_bytes": 2_245_632, "weights": 4096 * 4096,
                       "mfma_insts": 38_912, "valu_insts": 1_597_728, "lds_insts": 100_640,
                       "lds_bank_conflict_cycles": 219_200},
    # one M = 1 call on a 28672 x 8192 weight (the gate shape of the 70B-class model)
    "gemv_stream": {"source": "bit_nf4_quantized_dq_amd/csrc/gemv_stream.hip",
                    "sha1": "582116b2f7d814e3398559b0f16316fbc13952b6",
                    "read_bytes": 123_147_008, "write_bytes": 361_984, "weights": 28672 * 8192,
                    "mfma_insts": 459_648, "valu_insts": 6_625_632, "lds_insts": 2_429_888,
                    "lds_bank_conflict_cycles": 344_064},
    # the decode-once forward at M = 2048 on the same 28672 x 8192 weight: the decode (with
    # T = X A^T) and the BF16 GEMM
    "fwd_prologue_gate_M2048": {"source": "bit_nf4_quantized_dq_amd/csrc/lora.hip",
                                "sha1": "0b8df2d485634ad8f60dc2dba058b04007f6deeb",
                                "read_bytes": 157_554_176, "write_bytes": 469_827_584},
    "gemm_nt_gate_M2048": {"source": "bit_nf4_quantized_dq_amd/csrc/gemm_nt.hip",
                           "sha1": "5ce5dbfd0aa38821b99f12d226e7a0e43790f4b7",
                           "read_bytes": 2_001_885_389, "write_bytes": 117_440_512,
                           "mfma_insts": 29_532_160, "mfma_busy_cycles": 945_029_120},
}
SIMDS = 256 * 4  # MFMA pipes on the chip


def _counter_record(kernel):
    import hashlib

    rec = COUNTERS[kernel]
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), rec["source"])
    try:
        with open(path, "rb") as f:
            if hashlib.sha1(f.read()).hexdigest() != rec["sha1"]:
                return None
    except OSError:
        return None
    return rec


def counter_traffic(kernel):
    if kernel not in COUNTERS:
        return None
    rec = _counter_record(kernel)
    return None if rec is None else rec["read_bytes"] + rec["write_bytes"]


def counter_figures(kernel, avg_us=None):
    """The pinned counters of one launch, with what follows from them: VALU lane-ops per
    weight (wave instructions x 64 lanes, MFMA included: an upper bound, as masked-off lanes
    count) and, given the launch time, the fraction of it the MFMA pipes were busy at the
    published 2.4 GHz clock."""
    rec = _counter_record(kernel) if kernel in COUNTERS else None
    if rec is None:
        return None
    out = {k: v for k, v in rec.items() if k not in ("source", "sha1")}
    if "weights" in rec:
        out["valu_lane_ops_per_weight"] = round(64 * rec["valu_insts"] / rec["weights"], 3)
        out["valu_lane_ops_per_weight_excl_mfma"] = round(64 * (rec["valu_insts"] - rec["mfma_insts"]) / rec["weights"], 3)
    if "mfma_busy_cycles" in rec:
        out["mfma_busy_cycles_per_simd"] = rec["mfma_busy_cycles"] // SIMDS
        out["mfma_cycles_per_inst"] = round(rec["mfma_busy_cycles"] / rec["mfma_insts"], 2)
        if avg_us:
            out["mfma_busy_frac_at_2p4GHz"] = round(rec["mfma_busy_cycles"] / SIMDS / (avg_us * 2400.0), 4)
    return out


EVENT_STEPS = 4  # timed steps whose GEMM launches carry HIP events
WINDOWS = 20     # timed windows (step boundaries with events) for the median step time


class HipEvents:
    """Timing-only HIP events (no system-scope fence on record, so no L2 write-back around
    them) from the HIP runtime this process already runs (the one torch loaded)."""

    def __init__(self, n):
        import ctypes

        path = next((ln.split()[-1] for ln in open("/proc/self/maps") if "libamdhip64.so" in ln), None)
        if path is None:
            raise RuntimeError("HIP runtime not loaded")
        self.L = ctypes.CDLL(path)
        self.ct = ctypes
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.L.hipEventCreateWithFlags(ctypes.byref(e), ctypes.c_uint(0x20000000)) != 0:  # DisableSystemFence
                raise RuntimeError("hipEventCreateWithFlags failed")
            self.ev.append(e)

    def record(self, i, stream_ptr):
        if self.L.hipEventRecord(self.ev[i], self.ct.c_void_p(stream_ptr)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def ms(self, i, j):
        f = self.ct.c_float()
        self.L.hipEventSynchronize(self.ev[j])
        if self.L.hipEventElapsedTime(self.ct.byref(f), self.ev[i], self.ev[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return f.value

    def close(self):
        for e in self.ev:
            self.L.hipEventDestroy(e)


def step_flops(M, N, K, r):
    return 4 * M * N * K + 6 * M * r * (N + K)


def stream_bytes(M, N, K, r):
    # 0.515869 B/weight of NF4+DQ (codes, code8, c2s, mu) + adapters + activations
    return N * K // 2 + N * K // 64 + 4 * ((N * K // 64 + 255) // 256) + 4 + 2 * r * (N + K) + 2 * M * K + 2 * M * N


def merge_bytes(N, K, r):
    # NF4+DQ weight read + both adapters read + the BF16 merged weight written
    return N * K // 2 + N * K // 64 + 4 * ((N * K // 64 + 255) // 256) + 4 + 2 * r * (N + K) + 2 * N * K


def llama3_8b_layer(dev, steps=5, warmup=3):
    """Llama-3-8B-shaped decoder layer: all seven linears (q, k, v, o, gate, up, down), LoRA
    r = 16 on each, M = 8192 tokens; a step is the seven forwards then the seven backwards."""
    import torch

    import bit_nf4_quantized_dq_amd as Q
    from bit_nf4_quantized_dq_amd import inputs as I

    M, r, alpha = 8192, 16, 32.0
    lin, flops, wsf, wsb = [], 0, 0, 0
    for idx, shp in enumerate(I.LLAMA3_8B_LAYER):
        N, K = shp.d_out, shp.d_in
        W = I.weight(4, idx, N, K, 0.02, device=dev)
        q = Q.quantize(W)
        del W
        t = dict(q=q, X=I.activations(4, idx, M, K, device=dev), dY=I.grad_out(4, idx, M, N, device=dev),
                 A=I.lora_A(4, idx, r, K, device=dev), B=I.lora_B(4, idx, N, r, device=dev),
                 Y=torch.empty(M, N, dtype=torch.bfloat16, device=dev), T=torch.empty(M, r, dtype=torch.bfloat16, device=dev),
                 dX=torch.empty(M, K, dtype=torch.bfloat16, device=dev), dA=torch.empty(r, K, dtype=torch.bfloat16, device=dev),
                 dB=torch.empty(N, r, dtype=torch.bfloat16, device=dev))
        lin.append(t)
        flops += step_flops(M, N, K, r)
        wsf = max(wsf, Q.workspace_size(Q.OP_FWD, M, N, K, r))
        wsb = max(wsb, Q.workspace_size(Q.OP_BWD, M, N, K, r))
    ws_f = Q.new_workspace(wsf, dev)
    ws_b = Q.new_workspace(wsb, dev)

    def step():
        for t in lin:
            Q.linear_fwd(t["q"], t["X"], t["A"], t["B"], alpha, Y=t["Y"], T_save=t["T"], ws=ws_f)
        for t in reversed(lin):
            Q.linear_bwd(t["q"], t["X"], t["dY"], t["A"], t["B"], alpha, T_saved=t["T"], dX=t["dX"], dA=t["dA"],
                         dB=t["dB"], ws=ws_b)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = 1e3 * (time.perf_counter() - t0) / steps
    return {"metric": "NF4+DQ decoder-layer linears fwd+bwd TFLOP/s (7 linears, M=8192, r=16)",
            "value": round(flops / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "ms_per_step": round(ms, 3),
            "step_tflop": round(flops / 1e12, 4), "steps": steps,
            "roofline_frac": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}


def llama3_8b_mlp(dev, steps=5, warmup=3):
    """Llama-3-8B-shaped MLP block (gate and up 14336x4096, down 4096x14336, NF4+DQ, LoRA
    r = 16 on each) at M = 8192 tokens: one forward, then the backward through the block,
    with the forward's G and U kept (saved) or recomputed from X (checkpointing).  The rate
    counts the three linears' forward and backward FLOPs; the recompute's two extra
    projections are reported separately."""
    import torch

    import bit_nf4_quantized_dq_amd as Q
    from bit_nf4_quantized_dq_amd import inputs as I

    M, r, alpha, d, f = 8192, 16, 32.0, 4096, 14336
    shapes = [(f, d), (f, d), (d, f)]
    qs, As, Bs = [], [], []
    for i, (N, K) in enumerate(shapes):
        W = I.weight(6, 40 + i, N, K, 0.02, device=dev)
        qs.append(Q.quantize(W))
        del W
        As.append(I.lora_A(6, 40 + i, r, K, device=dev))
        Bs.append(I.lora_B(6, 40 + i, N, r, device=dev))
    X = I.activations(6, 49, M, d, device=dev)
    dY = I.grad_out(6, 49, M, d, device=dev)
    Y = torch.empty(M, d, dtype=torch.bfloat16, device=dev)
    dX = torch.empty(M, d, dtype=torch.bfloat16, device=dev)
    G = torch.empty(M, f, dtype=torch.bfloat16, device=dev)
    U = torch.empty(M, f, dtype=torch.bfloat16, device=dev)
    ws_f = Q.new_workspace(Q.mlp_workspace_size(Q.OP_FWD, M, *qs, r), dev)
    ws_b = Q.new_workspace(Q.mlp_workspace_size(Q.OP_BWD, M, *qs, r), dev)
    flops = sum(step_flops(M, N, K, r) for N, K in shapes)
    out = {"metric": "NF4+DQ MLP block fwd+bwd TFLOP/s (gate/up 14336x4096, down 4096x14336, M=8192, r=16)",
           "unit": "TFLOP/s", "step_tflop": round(flops / 1e12, 4), "steps": steps}
    for key, saved in (("saved", True), ("recompute", False)):
        def step():
            Q.mlp_fwd(qs, X, As, Bs, alpha, Y=Y, G_save=G if saved else None, U_save=U if saved else None, ws=ws_f)
            Q.mlp_bwd(qs, X, dY, As, Bs, alpha, G_saved=G if saved else None, U_saved=U if saved else None, dX=dX,
                      ws=ws_b)

        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        ms = 1e3 * (time.perf_counter() - t0) / steps
        out[key] = {"value": round(flops / (ms * 1e-3) / 1e12, 2), "ms_per_step": round(ms, 3),
                    "roofline_frac": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    del qs, As, Bs, X, dY, Y, dX, G, U, ws_f, ws_b
    torch.cuda.empty_cache()
    return out


def seventy_b_model(dev, layers=80, passes=3):
    """70B-class model: 80 layers x 7 linears (q, o 8192^2; k, v 1024x8192; gate, up
    28672x8192; down 8192x28672), NF4+DQ resident on the GPU (~35 GB), LoRA r = 16 on every
    linear.  M = 1: one forward through all linears, captured once in a HIP graph and replayed
    (every call streams its own weights from HBM), first one call per linear, then with the
    linears that share an input (q, k, v and gate, up) as grouped launches.  M = 2048: one
    eager forward pass."""
    import torch

    import bit_nf4_quantized_dq_amd as Q
    from bit_nf4_quantized_dq_amd import inputs as I

    r, alpha = 16, 32.0
    lin, nbytes1, flops2048 = [], 0, 0
    for layer in range(layers):
        for idx, shp in enumerate(I.SEVENTY_B_LAYER):
            N, K = shp.d_out, shp.d_in
            W = I.weight(5, idx, N, K, 0.015, layer, device=dev)
            q = Q.quantize(W)
            del W
            lin.append((q, I.lora_A(5, idx, r, K, layer, device=dev), I.lora_B(5, idx, N, r, layer, device=dev)))
            nbytes1 += stream_bytes(1, N, K, r)
            flops2048 += 2 * 2048 * N * K + 2 * 2048 * r * (N + K)
    weights_gb = sum(q.nbytes() for q, _, _ in lin) / 1e9
    shapes = {(s.d_out, s.d_in) for s in I.SEVENTY_B_LAYER}
    out = {"weights_GB": round(weights_gb, 3), "linears": len(lin)}
    for M in (1, 2048):
        Xs = {K: I.activations(5, 99, M, K, device=dev) for _, K in shapes}
        Ys = [torch.empty(M, s.d_out, dtype=torch.bfloat16, device=dev) for s in I.SEVENTY_B_LAYER]
        need = max(Q.workspace_size(Q.OP_FWD, M, N, K, r) for N, K in shapes)
        groups = [[0, 1, 2], [3], [4, 5], [6]]  # q, k, v | o | gate, up | down: each group reads one input
        for grp_ in groups:
            if len(grp_) > 1:
                need = max(need, Q.workspace_size_multi([lin[i][0] for i in grp_], M, r))
        ws = Q.new_workspace(need, dev)

        def fwd_pass():
            for i, (q, A, B) in enumerate(lin):
                Q.linear_fwd(q, Xs[q.d_in], A, B, alpha, Y=Ys[i % 7], ws=ws)

        def fwd_pass_grouped():
            for layer in range(layers):
                base = 7 * layer
                for grp_ in groups:
                    if len(grp_) == 1:
                        q, A, B = lin[base + grp_[0]]
                        Q.linear_fwd(q, Xs[q.d_in], A, B, alpha, Y=Ys[grp_[0]], ws=ws)
                    else:
                        qs = [lin[base + i][0] for i in grp_]
                        Q.linear_fwd_multi(qs, Xs[qs[0].d_in], [lin[base + i][1] for i in grp_],
                                           [lin[base + i][2] for i in grp_], alpha, Ys=[Ys[i] for i in grp_], ws=ws)

        fwd_pass()
        torch.cuda.synchronize()
        if M == 1:
            fwd_pass_grouped()
            torch.cuda.synchronize()
            for key, fn, what in (("M1", fwd_pass, "one launch per linear"),
                                  ("M1_grouped", fwd_pass_grouped, "q/k/v and gate/up as grouped launches")):
                g = torch.cuda.CUDAGraph()
                cap = torch.cuda.Stream()
                cap.wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(cap):
                    with torch.cuda.graph(g, stream=cap):
                        fn()
                torch.cuda.synchronize()
                g.replay()
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                for _ in range(passes):
                    g.replay()
                torch.cuda.synchronize()
                ms = 1e3 * (time.perf_counter() - t0) / passes
                out[key] = {"metric": f"weight-stream GB/s at M=1 through all 560 linears, {what} (graph replay)",
                            "value": round(nbytes1 / (ms * 1e-3) / 1e9, 1), "unit": "GB/s", "ms_per_pass": round(ms, 3),
                            "bytes_per_pass": nbytes1,
                            "frac_of_hbm_peak": round(nbytes1 / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
                del g
            out["M1"]["gate_28672x8192_call"] = {"algorithmic_bytes": stream_bytes(1, 28672, 8192, r),
                                                 "counter_bytes": counter_traffic("gemv_stream"),
                                                 "counters": counter_figures("gemv_stream")}
        else:
            t0 = time.perf_counter()
            for _ in range(passes):
                fwd_pass()
            torch.cuda.synchronize()
            ms = 1e3 * (time.perf_counter() - t0) / passes
            out["M2048"] = {"metric": "forward TFLOP/s at M=2048 through all 560 linears",
                            "value": round(flops2048 / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
                            "ms_per_pass": round(ms, 2), "tflop_per_pass": round(flops2048 / 1e12, 2),
                            "roofline_frac": round(flops2048 / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                            # counted traffic of the gate projection's two launches (decode with
                            # T, then the BF16 GEMM over 2048 x 8192 and the decoded 28672 x 8192)
                            "gate_28672x8192": {
                                "prologue_traffic": counter_traffic("fwd_prologue_gate_M2048"),
                                "gemm_traffic": counter_traffic("gemm_nt_gate_M2048"),
                                "gemm_operand_bytes": 2 * (28672 * 8192 + 2048 * 8192) + 2 * 2048 * 28672,
                                "gemm_counters": counter_figures("gemm_nt_gate_M2048")}}
        del Xs, Ys, ws
    del lin
    torch.cuda.empty_cache()
    return out


def weight_stream(copies, X_all, A, B, alpha, N, K, r, M, dev, kernel, replays=20):
    """Forward of one linear at M tokens over rotated quantized copies (every call reads its
    weight from HBM): the calls back to back, captured once in a HIP graph, replayed
    `replays` times; median and spread of the per-call time over the replays, plus per-launch
    event durations of an eager pass for reference."""
    import torch

    import bit_nf4_quantized_dq_amd as Q

    X1 = X_all[:M].to(dev).contiguous()
    Y1 = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    ws1 = Q.new_workspace(Q.workspace_size(Q.OP_FWD, M, N, K, r), dev)
    for cp in copies[:8]:
        Q.linear_fwd(cp, X1, A, B, alpha, Y=Y1, ws=ws1)
    torch.cuda.synchronize()
    # (a) kernel durations from HIP events, eager launches
    Q.timing_enable(True)
    for cp in copies:
        Q.linear_fwd(cp, X1, A, B, alpha, Y=Y1, ws=ws1)
    torch.cuda.synchronize()
    gv_ms, gv_n = Q.timing_read("gemv_fwd")
    Q.timing_enable(False)
    # (b) whole calls back to back, captured once in a HIP graph and replayed
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            for cp in copies:
                Q.linear_fwd(cp, X1, A, B, alpha, Y=Y1, ws=ws1)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    per_call = []
    for _ in range(replays):
        t0 = time.perf_counter()
        graph.replay()
        torch.cuda.synchronize()
        per_call.append(1e6 * (time.perf_counter() - t0) / len(copies))
    per_call.sort()
    us_call = per_call[len(per_call) // 2]
    # (c) eager Python calls, for reference
    t0 = time.perf_counter()
    for cp in copies:
        Q.linear_fwd(cp, X1, A, B, alpha, Y=Y1, ws=ws1)
    torch.cuda.synchronize()
    us_eager = 1e6 * (time.perf_counter() - t0) / len(copies)
    del graph
    sb = stream_bytes(M, N, K, r)
    gemv_us = 1e3 * gv_ms / max(gv_n, 1)
    return {
        "metric": f"weight-stream GB/s at M={M} ({N}x{K}, r={r}, {len(copies)} rotated copies, HIP-graph replay)",
        "value": round(sb / (us_call * 1e-6) / 1e9, 1), "unit": "GB/s", "us_per_call": round(us_call, 2),
        "us_per_call_min": round(per_call[0], 2), "us_per_call_max": round(per_call[-1], 2), "replays": replays,
        "us_per_call_eager_python": round(us_eager, 2),
        "bytes_per_call": sb,
        # the kernel's roofline from the graph replay (back-to-back calls; the gaps between
        # launches are included, so this bounds the kernel time from above).  Per-launch events
        # add about 2 us to every launch they bracket, so their figure is kept for reference.
        "gemv_kernel": {"avg_us": round(us_call, 2), "achieved_GBs": round(sb / (us_call * 1e-6) / 1e9, 1),
                        "peak_GBs": PEAK_HBM_GBS, "frac": round(sb / (us_call * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                        "method": f"graph replay of {len(copies)} calls, median of {replays} replays, "
                                  "launch gaps included",
                        "avg_us_per_launch_events": round(gemv_us, 2),
                        "kernel": "k_" + kernel.split("_M")[0], "traffic": counter_traffic(kernel),
                        "counters": counter_figures(kernel)},
    }


def host_info():
    """CPU model, logical CPUs and RAM of the host that runs the oracle."""
    model, ram = "unknown", None
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), model)
        with open("/proc/meminfo") as f:
            kb = next((int(ln.split()[1]) for ln in f if ln.startswith("MemTotal")), None)
            ram = None if kb is None else round(kb / 2**20, 1)
    except OSError:
        pass
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "ram_GiB": ram}


def cpu_baseline(N, K, r, alpha, target_s=15.0):
    """The oracle as it stands, on the host cores: dequantize + fwd + bwd on a token sample,
    with the BLAS threads it uses by default, and once more on one thread."""
    import numpy as np

    import oracle as O
    from bit_nf4_quantized_dq_amd import inputs as I

    c = I.linear_case(3, 0, N, K, 4096, r, 0.02)
    oq = O.quantize(c["W"].numpy())
    Ms = 256
    X = c["X"][:Ms].float().numpy().astype(np.float64)
    dY = c["dY"][:Ms].float().numpy().astype(np.float64)
    A = c["A"].float().numpy().astype(np.float64)
    B = c["B"].float().numpy().astype(np.float64)

    def run(budget_s, max_n):
        t0 = time.perf_counter()
        n = 0
        while True:
            what = O.dequantize_f64(oq)
            O.lora_fwd(what, X, A, B, alpha, r)
            O.lora_bwd(what, X, dY, A, B, alpha, r)
            n += 1
            if time.perf_counter() - t0 > budget_s or n >= max_n:
                return n, (time.perf_counter() - t0) / n

    try:
        from threadpoolctl import threadpool_info, threadpool_limits

        threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:  # noqa: BLE001
        threadpool_limits, threads = None, os.cpu_count() or 1
    n, dt = run(target_s / 2, 8)
    single = None
    if threadpool_limits is not None:
        with threadpool_limits(limits=1, user_api="blas"):
            n1, dt1 = run(target_s / 2, 2)
        single = {"value": step_flops(Ms, N, K, r) / dt1 / 1e12, "s_per_step": round(dt1, 3), "steps": n1}
    return {
        "value": step_flops(Ms, N, K, r) / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{n} oracle step(s) (dequantize + FP64 fwd + bwd) at M={Ms} tokens of the {N}x{K} r={r} linear; "
                  f"{dt:.2f} s per step",
        "single_thread": single,
        "host": {**host_info(), "blas_threads": int(threads)},
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the Llama-3-8B layer and 70B-class model workloads")
    ap.add_argument("--pmc-pass", action="store_true",
                    help="run 2 steps, one merge, one AdamW step, two M = 1 and two M = 16 calls on the step's "
                         "weight, two M = 1 calls on a 28672x8192 weight and a plain 256 MiB device copy (the "
                         "counter calibration), print nothing")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); "
              "the library has no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import torch

    import bit_nf4_quantized_dq_amd as Q
    from bit_nf4_quantized_dq_amd import inputs as I

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    N = K = 4096
    M, r, alpha = 4096, 16, 32.0

    # ---- training step workload (inputs resident in HBM)
    c = I.linear_case(3, 0, N, K, M, r, 0.02, device="cpu")
    W = c["W"].to(dev)
    X, A, B, dY = (c[k].to(dev) for k in ("X", "A", "B", "dY"))
    q = Q.quantize(W)
    Y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    T = torch.empty(M, r, dtype=torch.bfloat16, device=dev)
    dX = torch.empty(M, K, dtype=torch.bfloat16, device=dev)
    dA = torch.empty(r, K, dtype=torch.bfloat16, device=dev)
    dB = torch.empty(N, r, dtype=torch.bfloat16, device=dev)
    ws_f = Q.new_workspace(Q.workspace_size(Q.OP_FWD, M, N, K, r), dev)
    ws_b = Q.new_workspace(Q.workspace_size(Q.OP_BWD, M, N, K, r), dev)

    def step():
        Q.linear_fwd(q, X, A, B, alpha, Y=Y, T_save=T, ws=ws_f)
        Q.linear_bwd(q, X, dY, A, B, alpha, T_saved=T, dX=dX, dA=dA, dB=dB, ws=ws_b)

    if args.pmc_pass:
        step()
        step()
        wm = torch.empty(N, K, dtype=torch.bfloat16, device=dev)
        Q.merge(q, A, B, alpha, out=wm)
        del wm
        na = I.LLAMA3_8B_ADAPTER_PARAMS
        st = [t.to(dev) for t in I.optimizer_state(1, na)]
        Q.adamw_step(st[0], st[1], st[2], st[3], 1, 2e-4, weight_decay=0.01,
                     param=torch.empty(na, dtype=torch.bfloat16, device=dev))
        del st
        # the step's own 4096 x 4096 weight at M = 1 and M = 16 (two calls each)
        for m in (1, 16):
            for _ in range(2):
                Q.linear_fwd(q, X[:m], A, B, alpha)
        # one large-weight stream call pair at M = 1 (a 28672 x 8192 gate-shaped linear)
        Wg = I.weight(5, 4, 28672, 8192, 0.015, device=dev)
        qg = Q.quantize(Wg)
        del Wg
        Xg = I.activations(5, 4, 1, 8192, device=dev)
        Ag, Bg = I.lora_A(5, 4, r, 8192, device=dev), I.lora_B(5, 4, 28672, r, device=dev)
        for _ in range(2):
            Q.linear_fwd(qg, Xg, Ag, Bg, alpha)
        # the decode-once path at M = 2048 on the same weight, and on a 1024 x 8192 one (the k
        # and v shape of the 70B-class model, whose product takes the split reduction)
        X2k = I.activations(5, 5, 2048, 8192, device=dev)
        Q.linear_fwd(qg, X2k, Ag, Bg, alpha)
        del qg
        Wk = I.weight(5, 6, 1024, 8192, 0.015, device=dev)
        qk = Q.quantize(Wk)
        del Wk
        Q.linear_fwd(qk, X2k, Ag, I.lora_B(5, 6, 1024, r, device=dev), alpha)
        del qk, X2k
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        return

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: exactly `steps` steps.  HIP events (timing-only, no system fence) around
    # the two GEMM launches of the last EVENT_STEPS steps: each recorded event costs the
    # stream about 5 us of command processing, so the other steps run without them.
    gemms = ("gemm_fwd", "gemm_dx")
    ev_from = max(0, args.steps - EVENT_STEPS)
    # window boundaries: about WINDOWS windows of whole steps, one timing-only event each
    per_win = max(1, args.steps // WINDOWS)
    bounds = list(range(0, args.steps, per_win))[:WINDOWS] + [args.steps]
    wev = HipEvents(len(bounds))
    sptr = torch.cuda.current_stream().cuda_stream
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if i == ev_from:
            Q.timing_enable(True, kernels=gemms)
        if i in bounds:
            wev.record(bounds.index(i), sptr)
        step()
    wev.record(len(bounds) - 1, sptr)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    win_ms = sorted(wev.ms(k, k + 1) / (bounds[k + 1] - bounds[k]) for k in range(len(bounds) - 1))
    wev.close()
    gemm_us = {}
    for name in gemms:
        ms, n = Q.timing_read(name)
        gemm_us[name] = 1e3 * ms / max(n, 1)
    Q.timing_enable(False)
    ms_per_step = 1e3 * (t1 - t0) / args.steps
    flops = step_flops(M, N, K, r)
    value = flops / (ms_per_step * 1e-3) / 1e12
    win_med = win_ms[len(win_ms) // 2]
    windows = {"windows": len(win_ms), "steps_per_window": per_win, "ms_per_step_median": round(win_med, 4),
               "ms_per_step_min": round(win_ms[0], 4), "ms_per_step_max": round(win_ms[-1], 4),
               "tflops_at_median": round(flops / (win_med * 1e-3) / 1e12, 2),
               "method": "timing-only HIP events at window boundaries inside the timed steps"}

    # separate pass with events on every launch: per-kernel breakdown (slower step)
    inst_steps = min(args.steps, 20)
    Q.timing_enable(True)
    for _ in range(inst_steps):
        step()
    torch.cuda.synchronize()
    per_kernel = {}
    # launches of the step whose HBM traffic was counted (the paired prologues and dA + dB)
    counted = {"dequant": "fwd_prologue", "dequant_t": "bwd_prologue", "lora_grad": "lora_grad2"}
    for name in Q.KERNEL_IDS:
        ms, n = Q.timing_read(name)
        if n:
            per_kernel[name] = {"avg_us": 1e3 * ms / n, "launches_per_step": n / inst_steps}
            tb = counter_traffic(counted[name]) if name in counted else None
            if tb:
                per_kernel[name]["traffic"] = tb
                per_kernel[name]["traffic_GBs"] = tb / (1e3 * ms / n) / 1e3
    Q.timing_enable(False)

    # dominant kernel roofline (algorithmic FLOPs per launch / avg launch time in the timed region)
    kflops = {"gemm_fwd": 2 * M * N * K + 2 * M * N * r, "gemm_dx": 2 * M * N * K + 2 * M * K * r}
    dom = max(kflops, key=lambda k: gemm_us[k])
    ach = kflops[dom] / (gemm_us[dom] * 1e-6) / 1e12
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(ach, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": counter_traffic("gemm_nt"),
                "traffic_algorithmic_bytes": 2 * (N * K + M * K + M * r + N * r) + 2 * M * N,
                "algorithmic_flops_per_launch": kflops[dom], "avg_us": round(gemm_us[dom], 2),
                "other_gemm_avg_us": {k: round(v, 2) for k, v in gemm_us.items() if k != dom},
                "counters": counter_figures("gemm_nt", gemm_us[dom])}

    # ---- weight stream at M = 1 and M = 16 over 128 distinct copies (>= 1.1 GB, beyond the
    # 256 MB cache)
    ncopy = 128
    base = Q.quantize(W)
    copies = [Q.QuantizedWeight(base.codes.clone(), base.code8.clone(), base.c2s.clone(), base.mu.clone(), N, K)
              for _ in range(ncopy)]
    del base
    stream = weight_stream(copies, c["X"], A, B, alpha, N, K, r, 1, dev, "gemv_rows_M1")
    stream16 = weight_stream(copies, c["X"], A, B, alpha, N, K, r, 16, dev, "gemv_fused_M16")

    # ---- merged export bf16(w_hat + s B A): the same rotated copies, 8 rotated outputs
    # (8 x 32 MiB, beyond the 256 MB cache)
    outs = [torch.empty(N, K, dtype=torch.bfloat16, device=dev) for _ in range(8)]
    for i in range(8):
        Q.merge(copies[i], A, B, alpha, out=outs[i])
    torch.cuda.synchronize()
    Q.timing_enable(True, kernels=("merge",))
    t0 = time.perf_counter()
    for i, cp in enumerate(copies):
        Q.merge(cp, A, B, alpha, out=outs[i % 8])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    mg_ms, mg_n = Q.timing_read("merge")
    Q.timing_enable(False)
    mb = merge_bytes(N, K, r)
    mg_ev_us = 1e3 * mg_ms / max(mg_n, 1)
    # kernel time from a graph replay of the same back-to-back calls (per-launch events add
    # about 2 us to every launch they bracket; the replay's launch gaps are a fraction of a us)
    mgraph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(mgraph, stream=cap):
            for i, cp in enumerate(copies):
                Q.merge(cp, A, B, alpha, out=outs[i % 8])
    torch.cuda.synchronize()
    mgraph.replay()
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for _ in range(4):
        mgraph.replay()
    torch.cuda.synchronize()
    mg_us = 1e6 * (time.perf_counter() - t2) / (4 * len(copies))
    del mgraph
    merge = {"bytes_per_call": mb, "traffic": counter_traffic("merge"), "kernel_avg_us": round(mg_us, 2),
             "achieved_GBs": round(mb / (mg_us * 1e-6) / 1e9, 1), "peak_GBs": PEAK_HBM_GBS,
             "frac": round(mb / (mg_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
             "method": "graph replay of 128 back-to-back calls, launch gaps included",
             "avg_us_per_launch_events": round(mg_ev_us, 2),
             "us_per_call_eager_python": round(1e6 * (t1 - t0) / len(copies), 2)}
    # context: a plain device copy moving the same kind of mixed read + write traffic
    src32 = torch.empty(32 << 20, dtype=torch.uint8, device=dev).fill_(1)
    cps = [torch.empty_like(src32) for _ in range(8)]
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(64):
        cps[i % 8].copy_(src32)
    e1.record()
    torch.cuda.synchronize()
    cp_us = 1e3 * e0.elapsed_time(e1) / 64
    merge["reference_device_copy_32MiB"] = {"us": round(cp_us, 2), "GBs_read_plus_write": round(2 * (32 << 20) / (cp_us * 1e-6) / 1e9, 1)}
    del outs, cps, src32
    del copies

    # ---- adapter optimizer step over the pages' 41.9M-parameter adapter set (one flat call)
    na = I.LLAMA3_8B_ADAPTER_PARAMS
    st_master, st_m, st_v, st_g = (t.to(dev) for t in I.optimizer_state(1, na))
    st_p = torch.empty(na, dtype=torch.bfloat16, device=dev)
    for t in range(1, 3):
        Q.adamw_step(st_master, st_m, st_v, st_g, t, 2e-4, weight_decay=0.01, param=st_p)
    torch.cuda.synchronize()
    Q.timing_enable(True, kernels=("adamw",))
    t0 = time.perf_counter()
    for t in range(3, 13):
        Q.adamw_step(st_master, st_m, st_v, st_g, t, 2e-4, weight_decay=0.01, param=st_p)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    aw_ms, aw_n = Q.timing_read("adamw")
    Q.timing_enable(False)
    aw_us = 1e3 * aw_ms / max(aw_n, 1)
    ab = 28 * na  # FP32 master, m, v read and written (24 B), BF16 grad read, BF16 weight written
    adamw = {"params": na, "bytes_per_call": ab, "traffic": counter_traffic("adamw"), "kernel_avg_us": round(aw_us, 2),
             "achieved_GBs": round(ab / (aw_us * 1e-6) / 1e9, 1), "peak_GBs": PEAK_HBM_GBS,
             "frac": round(ab / (aw_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
             "us_per_call_eager_python": round(1e6 * (t1 - t0) / 10, 2)}
    del st_master, st_m, st_v, st_g, st_p

    # ---- format study: every codebook x second-level format on the same Gaussian weight:
    # storage bits per weight, relative reconstruction MSE of the GPU's dequantized weight,
    # and the decode kernel's time (cache-warm, HIP events)
    study = {}
    w_ms = float(torch.mean(W.double() ** 2))
    for cb in Q.CODEBOOKS:
        for dqf in Q.DQ_FORMATS:
            qf = Q.quantize(W, codebook=cb, dq=dqf)
            wd = Q.dequantize(qf)
            Q.timing_enable(True, kernels=("dequant",))
            for _ in range(5):
                Q.dequantize(qf, out=wd)
            torch.cuda.synchronize()
            dms, dn = Q.timing_read("dequant")
            Q.timing_enable(False)
            nb = sum(Q.quant_sizes(N, K, dqf)) + (0 if dqf == "none" else 4)
            study[f"{cb}/{dqf}"] = {"bits_per_weight": round(8.0 * nb / (N * K), 4),
                                    "rel_mse": round(float(torch.mean((wd.double() - W.double()) ** 2)) / w_ms, 6),
                                    "dequant_us": round(1e3 * dms / max(dn, 1), 2)}
            del qf, wd

    # ---- quantize (load time) of the same FP32 weight
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    nq = 5
    for _ in range(nq):
        Q.quantize(W, out=q)
    torch.cuda.synchronize()
    q_ms = 1e3 * (time.perf_counter() - t0) / nq
    # the kernels alone (the call also synchronizes once to fold the mean on the host)
    Q.timing_enable(True, ["quant_pass1", "quant_pass2"])
    for _ in range(nq):
        Q.quantize(W, out=q)
    p1_ms, p1_n = Q.timing_read("quant_pass1")
    p2_ms, p2_n = Q.timing_read("quant_pass2")
    Q.timing_enable(False)
    p1_us = 1e3 * p1_ms / max(p1_n, 1)
    p1_bytes = N * K * 4 + N * K // 2 + N * K // 16  # FP32 in; codes and FP32 block constants out
    quant = {"ms": round(q_ms, 3), "input_GBs": round(4 * N * K / (q_ms * 1e-3) / 1e9, 1),
             "pass1_us": round(p1_us, 2), "pass1_GBs": round(p1_bytes / p1_us / 1e3, 1),
             "pass1_frac": round(p1_bytes / p1_us / 1e3 / PEAK_HBM_GBS, 4),
             "pass2_us": round(1e3 * p2_ms / max(p2_n, 1), 2)}

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "timed_windows": windows,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Gaussian W ~ N(0, 0.02^2), X ~ N(0,1), dY ~ N(0, 1e-2))",
        "config": {"workload": "nf4dq-lora-linear-4096x4096-M4096-r16-train (fwd + bwd dX, dA, dB)", "M": M, "d_out": N,
                   "d_in": K, "r": r, "alpha": alpha, "step_flops": flops},
        "roofline": roofline,
        "kernels_instrumented_pass": {k: {kk: round(vv, 3) for kk, vv in v.items()} for k, v in per_kernel.items()},
        "weight_stream_M1": stream,
        "weight_stream_M16": stream16,
        "quantize_4096x4096": quant,
        "merge_4096x4096": merge,
        "adamw_llama3_8b_adapters": adamw,
        "format_study_4096x4096": study,
    }
    if not args.no_extra:
        del q, W
        torch.cuda.empty_cache()
        out["llama3_8b_layer_M8192"] = llama3_8b_layer(dev)
        out["llama3_8b_mlp_block_M8192"] = llama3_8b_mlp(dev)
        torch.cuda.empty_cache()
        out["model_70b_class"] = seventy_b_model(dev)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(N, K, r, alpha)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
