"""The forward entry point that allocates nothing (qlora_linear_fwd_noalloc, for callers that
cannot allocate device memory) against the ordinary forward on a fresh workspace, called
through the C ABI: several calls in a row, the second on a smaller input than the first, each
output bit-equal to qlora_linear_fwd's (the same kernels and reduction split) and within the
oracle's tolerance; a call that needs more than the fixed scratch is refused before any
launch; calls captured in a HIP graph replay correctly."""

import numpy as np
import pytest
import torch

import oracle as O
from bit_nf4_quantized_dq_amd import inputs as I

pytestmark = pytest.mark.gpu
TOL = 1e-2


def _case(idx, N, K, M, r):
    from bit_nf4_quantized_dq_amd import quantize

    c = I.linear_case(17, idx, N, K, M, r, 0.02)
    q = quantize(c["W"].cuda())
    return c, q, {k: c[k].cuda() for k in ("X", "A", "B")}


def _f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _check_against_oracle(c, Y, T, alpha, r):
    what = O.dequantize_f64(O.quantize(c["W"].numpy()))
    Yr, Tr = O.lora_fwd(what, _f64(c["X"]), _f64(c["A"]), _f64(c["B"]), alpha, r)
    for got, ref in ((Y, Yr), (T, Tr)):
        assert float(np.max(np.abs(_f64(got) - ref)) / np.max(np.abs(ref))) <= TOL


def test_noalloc_forward_matches_the_workspace_forward(gpu_lib):
    from bit_nf4_quantized_dq_amd import linear_fwd, linear_fwd_noalloc

    # large first (split-K partials and counters over much of the scratch), then smaller ones
    shapes = [(4096, 4096, 16, 16), (272, 320, 3, 8), (1040, 4096, 300, 16), (4096, 4096, 1, 16), (8192, 4096, 2, 16)]
    for i, (N, K, M, r) in enumerate(shapes):
        print(f"noalloc {N}x{K} M={M} r={r}", flush=True)
        alpha = 2.0 * r
        c, q, t = _case(i, N, K, M, r)
        Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        T = torch.empty(M, r, dtype=torch.bfloat16, device="cuda")
        for rep in range(2):
            linear_fwd_noalloc(q, t["X"], t["A"], t["B"], alpha, Y, T_save=T)
            Tw = torch.empty_like(T)
            Yw = linear_fwd(q, t["X"], t["A"], t["B"], alpha, T_save=Tw)
            torch.cuda.synchronize()
            assert torch.equal(Y.view(torch.int16), Yw.view(torch.int16)), (N, K, M, rep)
            assert torch.equal(T.view(torch.int16), Tw.view(torch.int16)), (N, K, M, rep)
        if N * K <= (16 << 20):
            _check_against_oracle(c, Y, T, alpha, r)


def test_noalloc_refuses_calls_beyond_its_scratch(gpu_lib):
    from bit_nf4_quantized_dq_amd import QLoRAError, linear_fwd_noalloc

    c, q, t = _case(9, 4096, 4096, 1024, 16)
    Y = torch.zeros(1024, 4096, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(QLoRAError) as e:
        linear_fwd_noalloc(q, t["X"], t["A"], t["B"], 32.0, Y)
    assert e.value.status == -7
    torch.cuda.synchronize()
    assert int(Y.view(torch.int16).abs().sum()) == 0, "nothing was launched"


def test_noalloc_under_graph_capture(gpu_lib):
    """Captured calls (after the set-up call) replay with new inputs and match eager calls."""
    from bit_nf4_quantized_dq_amd import linear_fwd, linear_fwd_noalloc

    cases = []
    for i, (N, K, M, r) in enumerate([(4096, 4096, 1, 16), (272, 320, 16, 8), (1040, 4096, 64, 16)]):
        c, q, t = _case(20 + i, N, K, M, r)
        Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        linear_fwd_noalloc(q, t["X"], t["A"], t["B"], 2.0 * r, Y)
        cases.append((q, t, Y, 2.0 * r))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            for q, t, Y, alpha in cases:
                linear_fwd_noalloc(q, t["X"], t["A"], t["B"], alpha, Y)
    torch.cuda.synchronize()
    gen = torch.Generator().manual_seed(5)
    for rep in range(3):
        for q, t, Y, alpha in cases:
            t["X"].copy_(torch.randn(t["X"].shape, generator=gen).to(torch.bfloat16))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for q, t, Y, alpha in cases:
            ref = linear_fwd(q, t["X"], t["A"], t["B"], alpha)
            torch.cuda.synchronize()
            assert torch.equal(Y.view(torch.int16), ref.view(torch.int16)), rep
