"""GPU parity of the MLP block (qlora_mlp_fwd / qlora_mlp_bwd): gate and up projections,
the SiLU-gated product, the down projection, and the backward through all three, each
projection NF4 + DQ with a LoRA adapter, against the oracle in FP64 (exact intermediates) on
the same seeded inputs and the oracle's own decoded weights.

Tolerances (normwise, max|got - ref| / max|ref|).  G and U are single projections of the
exact BF16 input X: 1e-2, as for one linear.  The block's output and gradients come after a
chain of BF16 tensors, the compute type the pages fix: BF16 keeps 8 significant bits, so
each rounding adds a relative 2^-8 at most, and the longest chains (to dX and the gate and
up adapter gradients) pass G, U, dH and the down projection's rank-r intermediate, dG or dU,
their own rank-r intermediate and the output: about seven roundings, 7 * 2^-8 = 2.7e-2 to
first order.  The block's tensors are held to 3e-2."""

import numpy as np
import pytest
import torch

import oracle as O
from bit_nf4_quantized_dq_amd import inputs as I

pytestmark = pytest.mark.gpu
TOL = 1e-2        # a single projection of the exact input
TOL_BLOCK = 3e-2  # after the block's chain of BF16 tensors (module docstring)


def _f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def normwise(got, ref):
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(got - ref)) / (den if den > 0 else 1.0))


def _block(cfg, d, f, M, r):
    """The block's weights (gate, up [f, d]; down [d, f]), adapters, X [M, d] and dY [M, d]."""
    shapes = [(f, d), (f, d), (d, f)]
    Ws = [I.weight(cfg, 30 + i, n, k, 0.02) for i, (n, k) in enumerate(shapes)]
    As = [I.lora_A(cfg, 30 + i, r, k) for i, (n, k) in enumerate(shapes)]
    Bs = [(I.lora_B(cfg, 30 + i, n, r).float() * 10).to(torch.bfloat16) for i, (n, k) in enumerate(shapes)]
    X = I.activations(cfg, 39, M, d)
    dY = I.grad_out(cfg, 39, M, d)
    return Ws, As, Bs, X, dY


@pytest.mark.parametrize("d,f,M,r", [
    (256, 512, 4, 8),      # M <= 16: weight-streaming kernels
    (256, 768, 64, 16),    # 16 < M < 1024: fused dequant GEMMs
    (512, 1024, 1100, 16), # M >= 1024: decoded copy + BF16 GEMM, ragged token tiles
])
@pytest.mark.parametrize("saved", [False, True])
def test_mlp_block_matches_oracle(gpu_lib, d, f, M, r, saved):
    from bit_nf4_quantized_dq_amd import mlp_bwd, mlp_fwd, quantize

    print(f"mlp d={d} f={f} M={M} r={r} saved={saved}", flush=True)
    alpha = 2.0 * r
    Ws, As, Bs, X, dY = _block(15, d, f, M, r)
    qs = [quantize(W.cuda()) for W in Ws]
    What = [O.bf16_bits_to_f32(O.dequantize_bf16_bits(O.quantize(W.numpy()))).astype(np.float64) for W in Ws]
    Ad, Bd = [a.cuda() for a in As], [b.cuda() for b in Bs]
    Xd, dYd = X.cuda(), dY.cuda()
    G = torch.empty(M, f, dtype=torch.bfloat16, device="cuda") if saved else None
    U = torch.empty(M, f, dtype=torch.bfloat16, device="cuda") if saved else None
    Y = mlp_fwd(qs, Xd, Ad, Bd, alpha, G_save=G, U_save=U)
    dX, dAs, dBs = mlp_bwd(qs, Xd, dYd, Ad, Bd, alpha, G_saved=G, U_saved=U)
    torch.cuda.synchronize()
    Af, Bf, Xf, dYf = [_f64(a) for a in As], [_f64(b) for b in Bs], _f64(X), _f64(dY)
    Y_ref, G_ref, U_ref, _ = O.mlp_fwd(What[0], What[1], What[2], Xf, Af, Bf, alpha, r)
    dX_ref, dA_ref, dB_ref = O.mlp_bwd(What[0], What[1], What[2], Xf, dYf, Af, Bf, alpha, r)
    assert normwise(_f64(Y), Y_ref) <= TOL_BLOCK
    if saved:
        assert normwise(_f64(G), G_ref) <= TOL and normwise(_f64(U), U_ref) <= TOL
    assert normwise(_f64(dX), dX_ref) <= TOL_BLOCK
    for i in range(3):
        assert normwise(_f64(dAs[i]), dA_ref[i]) <= TOL_BLOCK, f"dA[{i}]"
        assert normwise(_f64(dBs[i]), dB_ref[i]) <= TOL_BLOCK, f"dB[{i}]"


def test_mlp_recompute_equals_saved(gpu_lib):
    """The backward that recomputes G and U from X gives the same bits as the one handed the
    forward's saved G and U (same kernels, same inputs)."""
    from bit_nf4_quantized_dq_amd import mlp_bwd, mlp_fwd, quantize

    d, f, M, r = 512, 1024, 1024, 16
    Ws, As, Bs, X, dY = _block(16, d, f, M, r)
    qs = [quantize(W.cuda()) for W in Ws]
    Ad, Bd = [a.cuda() for a in As], [b.cuda() for b in Bs]
    Xd, dYd = X.cuda(), dY.cuda()
    G = torch.empty(M, f, dtype=torch.bfloat16, device="cuda")
    U = torch.empty(M, f, dtype=torch.bfloat16, device="cuda")
    mlp_fwd(qs, Xd, Ad, Bd, 32.0, G_save=G, U_save=U)
    a = mlp_bwd(qs, Xd, dYd, Ad, Bd, 32.0, G_saved=G, U_saved=U)
    b = mlp_bwd(qs, Xd, dYd, Ad, Bd, 32.0)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0])
    for i in range(3):
        assert torch.equal(a[1][i], b[1][i]) and torch.equal(a[2][i], b[2][i])


def test_mlp_block_decode_groups_gate_and_up(gpu_lib):
    """At decode size (M <= 16) with gate + up holding 32M weights or more, the forward runs
    gate and up as one grouped weight-streaming launch: the block's output, G and U against
    the oracle, and the backward at the same size, within the block tolerance."""
    from bit_nf4_quantized_dq_amd import mlp_bwd, mlp_fwd, quantize, timing_enable, timing_read

    d, f, M, r = 2048, 8192, 2, 16
    alpha = 32.0
    print(f"mlp decode d={d} f={f} M={M}", flush=True)
    Ws, As, Bs, X, dY = _block(17, d, f, M, r)
    qs = [quantize(W.cuda()) for W in Ws]
    What = [O.bf16_bits_to_f32(O.dequantize_bf16_bits(O.quantize(W.numpy()))).astype(np.float64) for W in Ws]
    Ad, Bd = [a.cuda() for a in As], [b.cuda() for b in Bs]
    G = torch.empty(M, f, dtype=torch.bfloat16, device="cuda")
    U = torch.empty(M, f, dtype=torch.bfloat16, device="cuda")
    timing_enable(True, ["gemv_fwd"])
    try:
        timing_read("gemv_fwd")
        Y = mlp_fwd(qs, X.cuda(), Ad, Bd, alpha, G_save=G, U_save=U)
        torch.cuda.synchronize()
        _, launches = timing_read("gemv_fwd")
    finally:
        timing_enable(False)
    assert launches == 2, "gate + up grouped, then down"
    dX, dAs, dBs = mlp_bwd(qs, X.cuda(), dY.cuda(), Ad, Bd, alpha, G_saved=G, U_saved=U)
    torch.cuda.synchronize()
    Af, Bf, Xf, dYf = [_f64(a) for a in As], [_f64(b) for b in Bs], _f64(X), _f64(dY)
    Y_ref, G_ref, U_ref, _ = O.mlp_fwd(What[0], What[1], What[2], Xf, Af, Bf, alpha, r)
    dX_ref, dA_ref, dB_ref = O.mlp_bwd(What[0], What[1], What[2], Xf, dYf, Af, Bf, alpha, r)
    assert normwise(_f64(G), G_ref) <= TOL and normwise(_f64(U), U_ref) <= TOL
    assert normwise(_f64(Y), Y_ref) <= TOL_BLOCK
    assert normwise(_f64(dX), dX_ref) <= TOL_BLOCK
    for i in range(3):
        assert normwise(_f64(dAs[i]), dA_ref[i]) <= TOL_BLOCK, f"dA[{i}]"
        assert normwise(_f64(dBs[i]), dB_ref[i]) <= TOL_BLOCK, f"dB[{i}]"
