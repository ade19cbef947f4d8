"""GPU parity of the grouped forward (qlora_linear_fwd_multi): several linears that read the
same activations, run as one weight-streaming launch when they qualify and as single calls
otherwise.  Each output is checked against the oracle (sampled rows, saved T in full) within
the forward tolerance, max|got - ref| / max|ref| <= 1e-2; the fallback path must equal the
single calls bit for bit, since it runs exactly those launches."""

import numpy as np
import pytest
import torch

import oracle as O
from bit_nf4_quantized_dq_amd import inputs as I

pytestmark = pytest.mark.gpu
TOL = 1e-2


def _f64(t_bf16):
    return t_bf16.detach().float().cpu().numpy().astype(np.float64)


def normwise(got, ref):
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(got - ref)) / (den if den > 0 else 1.0))


def _group(cfg, dims, K, M, r, std=0.02):
    """Weights, adapters and the one shared X of a group (linear i uses seed index 60 + i)."""
    X = I.activations(cfg, 59, M, K)
    ws = [I.weight(cfg, 60 + i, N, K, std) for i, N in enumerate(dims)]
    As = [I.lora_A(cfg, 60 + i, r, K) for i in range(len(dims))]
    Bs = [I.lora_B(cfg, 60 + i, N, r) for i, N in enumerate(dims)]
    return X, ws, As, Bs


GROUPS = [
    # d_outs, d_in, M, r
    ([8192, 1024, 1024], 4096, 1, 16),          # q, k, v shaped
    ([4096, 4096], 4096, 3, 40),                # gate + up shaped; B ranks past 32 read element by element
    ([2048, 1024, 1024, 256], 8192, 16, 128),   # four linears, M = 16, the largest rank
    ([7168, 1024], 4096, 2, 12),                # r not a multiple of 8
]


@pytest.mark.parametrize("dims,K,M,r", GROUPS)
def test_grouped_stream_matches_oracle(gpu_lib, dims, K, M, r):
    from bit_nf4_quantized_dq_amd import linear_fwd_multi, quantize, timing_enable, timing_read

    print(f"group {dims} x {K} M={M} r={r}", flush=True)
    alpha = 2.0 * r
    X, Ws, As, Bs = _group(11, dims, K, M, r)
    qs = [quantize(W.cuda()) for W in Ws]
    Ts = [torch.empty(M, r, dtype=torch.bfloat16, device="cuda") for _ in dims]
    timing_enable(True, ["gemv_fwd"])
    try:
        timing_read("gemv_fwd")
        Ys = linear_fwd_multi(qs, X.cuda(), [a.cuda() for a in As], [b.cuda() for b in Bs], alpha, T_saves=Ts)
        torch.cuda.synchronize()
        _, launches = timing_read("gemv_fwd")
    finally:
        timing_enable(False)
    assert launches == 1, "the group qualifies for one weight-streaming launch"
    Xf = _f64(X)
    rng = np.random.default_rng(sum(dims) + K + M + r)
    for i, (N, W) in enumerate(zip(dims, Ws)):
        n_s = np.unique(np.concatenate([rng.choice(N, min(N, 24), replace=False), np.arange(0, N, 256)[:6],
                                        [0, 255 % N, N - 1]]))
        mask = np.zeros((N, K // 64), bool)
        mask[n_s, :] = True
        oq = O.quantize(W.numpy(), blocks=mask)
        what = O.bf16_bits_to_f32(O.dequantize_bf16_bits(oq)[n_s]).astype(np.float64)
        Af, Bf = _f64(As[i]), _f64(Bs[i])
        T_ref = Xf @ Af.T
        Y_ref = Xf @ what.T + (alpha / r) * T_ref @ Bf[n_s].T
        assert normwise(_f64(Ys[i])[:, n_s], Y_ref) <= TOL, f"Y[{i}]"
        assert normwise(_f64(Ts[i]), T_ref) <= TOL, f"T[{i}]"


def test_grouped_stream_is_deterministic_and_replays(gpu_lib):
    """Two eager calls and three HIP-graph replays (new inputs copied in between) give the
    same bits: the group's arrival counters reset themselves."""
    from bit_nf4_quantized_dq_amd import linear_fwd_multi, new_workspace, quantize, workspace_size_multi

    dims, K, M, r = [8192, 1024, 1024], 4096, 1, 16
    X, Ws, As, Bs = _group(11, dims, K, M, r)
    qs = [quantize(W.cuda()) for W in Ws]
    Xd, Ad, Bd = X.cuda(), [a.cuda() for a in As], [b.cuda() for b in Bs]
    Ys = [torch.empty(M, N, dtype=torch.bfloat16, device="cuda") for N in dims]
    ws = new_workspace(workspace_size_multi(qs, M, r), "cuda")
    first = [y.clone() for y in linear_fwd_multi(qs, Xd, Ad, Bd, 32.0, Ys=Ys, ws=ws)]
    linear_fwd_multi(qs, Xd, Ad, Bd, 32.0, Ys=Ys, ws=ws)
    torch.cuda.synchronize()
    for a, b in zip(first, Ys):
        assert torch.equal(a, b)
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            linear_fwd_multi(qs, Xd, Ad, Bd, 32.0, Ys=Ys, ws=ws)
    torch.cuda.synchronize()
    for rep in range(3):
        X2 = I.activations(11, 70 + rep, M, K).cuda()
        Xd.copy_(X2)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [y.clone() for y in Ys]
        eager = linear_fwd_multi(qs, Xd, Ad, Bd, 32.0, ws=ws)
        torch.cuda.synchronize()
        for a, b in zip(got, eager):
            assert torch.equal(a, b), f"replay {rep}"


@pytest.mark.parametrize("dims,K,M,r", [
    ([1008, 512], 1024, 4, 8),        # d_out not a multiple of 256: single calls
    ([4096, 1024, 1024], 4096, 64, 16),  # M > 16: single calls of the fused GEMM
    ([2048, 2048], 4096, 1, 16),      # 16M weights in all: below the streaming threshold
    ([8192], 4096, 1, 16),            # a group of one: the single call
])
def test_grouped_fallback_equals_single_calls(gpu_lib, dims, K, M, r):
    from bit_nf4_quantized_dq_amd import linear_fwd, linear_fwd_multi, quantize

    print(f"fallback {dims} x {K} M={M} r={r}", flush=True)
    X, Ws, As, Bs = _group(12, dims, K, M, r)
    qs = [quantize(W.cuda()) for W in Ws]
    Xd, Ad, Bd = X.cuda(), [a.cuda() for a in As], [b.cuda() for b in Bs]
    Ts = [torch.empty(M, r, dtype=torch.bfloat16, device="cuda") for _ in dims]
    Ys = linear_fwd_multi(qs, Xd, Ad, Bd, 24.0, T_saves=Ts)
    for i, q in enumerate(qs):
        T1 = torch.empty(M, r, dtype=torch.bfloat16, device="cuda")
        Y1 = linear_fwd(q, Xd, Ad[i], Bd[i], 24.0, T_save=T1)
        torch.cuda.synchronize()
        assert torch.equal(Ys[i], Y1), f"Y[{i}]"
        assert torch.equal(Ts[i], T1), f"T[{i}]"
