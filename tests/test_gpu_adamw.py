"""GPU parity of the adapter optimizer step (AdamW, FP32 states, BF16 gradient and working
weight) through the C ABI against the CPU oracle.

Tolerance, derived from the arithmetic.  The library evaluates the update in FP32 with
every operation rounded once (u = 2^-24) and its step scalars rounded once from FP64:
  - m: three roundings over non-negative-weighted terms, |dm| <= 3u (b1 |m| + (1-b1) |g|);
  - v: four roundings over non-negative terms, relative error <= 4u;
  - the denominator sqrt(v) / sqrt(1-b2^t) + eps: relative error <= 0.5 * 4u + 3u = 5u;
  - the step U = lr / (1-b1^t) * m / den: |dU| <= |U| (5u + 4u) + lr/(1-b1^t) |dm| / den;
  - theta: decay (2u relative) and the final subtraction (u).
The tests allow 4x of each term:
  |d theta| <= 2^-21 (2 |theta| + 9 |U| + 3 lr/(1-b1^t) M / den),   M = b1 |m| + (1-b1) |g|,
  |d m| <= 2^-21 M + 2^-24 |m|,   |d v| <= 2^-20 (b2 v + (1-b2) g^2) + 2^-24 v.
The BF16 working weight may differ by one step only where the oracle's exact theta lies
within the theta tolerance of a BF16 rounding boundary.  Hyperparameters are handed to the
oracle as the FP32 values the C ABI receives."""

import numpy as np
import pytest
import torch

import oracle as O
from bit_nf4_quantized_dq_amd import inputs as I

pytestmark = pytest.mark.gpu
F32 = lambda x: float(np.float32(x))  # noqa: E731


def _bits(t):
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def _tols(master, m, v, g, t, lr, b1, b2, eps):
    th0 = master.astype(np.float64)
    m0, v0 = m.astype(np.float64), v.astype(np.float64)
    g = O.bf16_bits_to_f32(g).astype(np.float64)
    M = b1 * np.abs(m0) + (1 - b1) * np.abs(g)
    V = b2 * v0 + (1 - b2) * g * g
    m1 = b1 * m0 + (1 - b1) * g
    den = np.sqrt(V / (1 - b2**t)) + eps
    ss = lr / (1 - b1**t)
    U = ss * m1 / den
    tol_th = 2.0**-21 * (2 * np.abs(th0) + 9 * np.abs(U) + 3 * ss * M / den)
    return tol_th, 2.0**-21 * M, 2.0**-20 * V


def _check_step(got, ref, tols):
    (th_g, m_g, v_g, p_g), (th_r, m_r, v_r, p_r, th_exact) = got, ref
    tol_th, tol_m, tol_v = tols
    assert np.all(np.abs(th_g.astype(np.float64) - th_exact) <= tol_th + 2.0**-24 * np.abs(th_exact)), "master"
    assert np.all(np.abs(m_g.astype(np.float64) - m_r.astype(np.float64)) <= tol_m + 2.0**-24 * np.abs(m_r)), "m"
    assert np.all(np.abs(v_g.astype(np.float64) - v_r.astype(np.float64)) <= tol_v + 2.0**-24 * np.abs(v_r)), "v"
    if p_g is None:
        return
    diff = p_g != p_r
    if diff.any():
        fg, fr = O.bf16_bits_to_f32(p_g[diff]).astype(np.float64), O.bf16_bits_to_f32(p_r[diff]).astype(np.float64)
        ulp = np.spacing(np.abs(fr).astype(np.float32)).astype(np.float64) * 2.0**16
        assert np.all(np.abs(fg - fr) <= ulp), "working weight off by more than one BF16 step"
        mid = 0.5 * (fg + fr)
        assert np.all(np.abs(mid - th_exact[diff]) <= 2 * tol_th[diff] + 2.0**-23 * np.abs(th_exact[diff]))
        assert diff.sum() <= max(4, diff.size // 1000)


def _run(n, seed, step, lr, b1, b2, eps, wd, with_param=True):
    master, m, v, grad = I.optimizer_state(seed, n)
    gbits = _bits(grad)
    ref = O.adamw_step(master.numpy(), m.numpy(), v.numpy(), gbits, step, lr, b1, b2, eps, wd)
    tols = _tols(master.numpy(), m.numpy(), v.numpy(), gbits, step, lr, b1, b2, eps)
    d = [x.cuda() for x in (master, m, v, grad)]
    p = torch.empty(n, dtype=torch.bfloat16, device="cuda") if with_param else None
    from bit_nf4_quantized_dq_amd import adamw_step

    adamw_step(d[0], d[1], d[2], d[3], step, lr, b1, b2, eps, wd, param=p)
    torch.cuda.synchronize()
    got = (d[0].cpu().numpy(), d[1].cpu().numpy(), d[2].cpu().numpy(), None if p is None else _bits(p))
    _check_step(got, ref, tols)
    return got


HP = dict(lr=F32(2e-4), b1=F32(0.9), b2=F32(0.999), eps=F32(1e-8), wd=F32(0.01))


@pytest.mark.parametrize("n", [1, 3, 4, 5, 1027, 1_000_003])
def test_adamw_parity_sizes(gpu_lib, n):
    print(f"adamw n={n}", flush=True)
    _run(n, 500 + n % 97, 1, **HP)


@pytest.mark.parametrize("step", [2, 10, 5000])
def test_adamw_parity_later_steps(gpu_lib, step):
    _run(65_537, 600 + step, step, **HP)


def test_adamw_degenerate_betas_and_no_param(gpu_lib):
    """b1 = b2 = 0: m = g and v = g^2, so the step is lr g / (|g| + eps)."""
    _run(4099, 700, 3, lr=F32(1e-3), b1=0.0, b2=0.0, eps=F32(1e-6), wd=F32(0.1), with_param=False)


def test_adamw_llama3_8b_adapter_set(gpu_lib):
    """The pages' 41.9M trainable parameters (r = 16 on every linear of the 8B model) in one
    call over the flat buffer."""
    n = I.LLAMA3_8B_ADAPTER_PARAMS
    print(f"adamw n={n}", flush=True)
    _run(n, 800, 1, **HP)


def test_adamw_three_steps_from_zero_state(gpu_lib):
    """Both sides run three steps from zero moments, each from its own previous state; the
    per-step bounds add up."""
    from bit_nf4_quantized_dq_amd import adamw_step

    n = 20_011
    master, _, _, _ = I.optimizer_state(900, n)
    th_r = master.numpy().copy()
    m_r = np.zeros(n, np.float32)
    v_r = np.zeros(n, np.float32)
    d_th, d_m, d_v = master.cuda(), torch.zeros(n, device="cuda"), torch.zeros(n, device="cuda")
    p = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    acc_tol, acc_m, acc_v = np.zeros(n), np.zeros(n), np.zeros(n)
    for t in range(1, 4):
        _, _, _, grad = I.optimizer_state(900 + t, n)
        gbits = _bits(grad)
        tol_th, tol_m, tol_v = _tols(th_r, m_r, v_r, gbits, t, HP["lr"], HP["b1"], HP["b2"], HP["eps"])
        acc_tol += tol_th + 2.0**-24 * np.abs(th_r)
        # earlier differences carry over, scaled by the decay of the moments
        acc_m = HP["b1"] * acc_m + tol_m + 2.0**-24 * np.abs(m_r)
        acc_v = HP["b2"] * acc_v + tol_v + 2.0**-24 * np.abs(v_r)
        th_r, m_r, v_r, p_r, th_exact = O.adamw_step(th_r, m_r, v_r, gbits, t, HP["lr"], HP["b1"], HP["b2"],
                                                      HP["eps"], HP["wd"])
        adamw_step(d_th, d_m, d_v, grad.cuda(), t, HP["lr"], HP["b1"], HP["b2"], HP["eps"], HP["wd"], param=p)
        torch.cuda.synchronize()
        # the states of the two sides drift apart by the accumulated rounding only
        g_th = d_th.cpu().numpy().astype(np.float64)
        assert np.all(np.abs(g_th - th_exact) <= 4 * acc_tol), f"step {t}"
        assert np.all(np.abs(d_m.cpu().numpy().astype(np.float64) - m_r) <= 2 * acc_m + 2.0**-24 * np.abs(m_r))
        assert np.all(np.abs(d_v.cpu().numpy().astype(np.float64) - v_r) <= 2 * acc_v + 2.0**-24 * np.abs(v_r))
    assert np.array_equal(_bits(p), O.bf16_round_bits(d_th.cpu().numpy()))


def test_adamw_zero_length_is_noop(gpu_lib):
    from bit_nf4_quantized_dq_amd import adamw_step

    e = torch.empty(0, device="cuda")
    adamw_step(e, e.clone(), e.clone(), torch.empty(0, dtype=torch.bfloat16, device="cuda"), 1, 1e-3)
    torch.cuda.synchronize()
