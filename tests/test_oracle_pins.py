"""Pins for the CPU oracle: each test checks the oracle against something other than
itself -- the pages' printed figures, closed forms, other libraries' routines, brute force
by a different formulation, or invariants the pages state.  CPU only."""

import json
import math
import os
import statistics

import numpy as np
import pytest
import scipy.special
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
GIB = float(2**30)


# ------------------------------------------------------------------ codebook

def test_codebook_shape_and_endpoints():
    q = O.nf4_codebook()
    assert q.dtype == np.float32 and q.shape == (16,)
    assert np.all(np.diff(q.astype(np.float64)) > 0), "levels strictly increasing"
    # exact zero with positive sign, exact endpoints (65B page, "NF4")
    assert q[8] == 0.0 and not np.signbit(q[8])
    assert q[0] == -1.0 and q[15] == 1.0
    assert np.sum(q < 0) == 8 and np.sum(q >= 0) == 8


def test_codebook_interior_antisymmetry():
    # q_i / q_{16-i} is one constant for i = 1..7 (literal formula, per-side scaling)
    ex = O.nf4_codebook_exact()
    ratios = [float(ex[i] / ex[16 - i]) for i in range(1, 8)]
    assert max(ratios) - min(ratios) < 1e-40
    raw15 = 0.5 * (statistics.NormalDist().inv_cdf(15 / 17) + statistics.NormalDist().inv_cdf(16 / 17))
    raw0 = statistics.NormalDist().inv_cdf(1 / 34)
    assert ratios[0] == pytest.approx(-raw15 / abs(raw0), rel=1e-12)


def _table_from(inv):
    raw = [inv(1 / 34)] + [0.5 * (inv(i / 17) + inv((i + 1) / 17)) for i in range(1, 16)]
    raw[8] = 0.0
    out = [raw[i] / -raw[0] for i in range(8)] + [0.0] + [raw[i] / raw[15] for i in range(9, 16)]
    return np.array(out, dtype=np.float64)


@pytest.mark.parametrize("which", ["statistics", "scipy"])
def test_codebook_matches_other_quantile_routines(which):
    """Two other inverse-normal routines (Wichura AS241 in `statistics`, cephes ndtri in
    SciPy) give the same FP32 table bit for bit."""
    inv = statistics.NormalDist().inv_cdf if which == "statistics" else (lambda p: float(scipy.special.ndtri(p)))
    t64 = _table_from(inv)
    q = O.nf4_codebook()
    assert np.max(np.abs(t64 - q.astype(np.float64))) < 2e-7
    assert np.array_equal(t64.astype(np.float32).view(np.uint32), q.view(np.uint32))


def test_codebook_levels_sit_in_their_quantile_bins():
    """Closed-form check through the CDF (math.erfc, not the oracle's erfinv): the
    un-normalised level i lies between Q(i/17) and Q((i+1)/17), and Phi(Q(j/17)) = j/17."""
    phi = lambda x: 0.5 * math.erfc(-x / math.sqrt(2.0))
    for j in range(1, 17):
        x = float(O.qlora_oracle._q_normal(j, 17))
        assert phi(x) == pytest.approx(j / 17, abs=1e-15)
    ex = O.nf4_codebook_exact()
    scale_pos = float(0.5 * (O.qlora_oracle._q_normal(15, 17) + O.qlora_oracle._q_normal(16, 17)))
    for i in range(9, 16):
        raw = float(ex[i]) * scale_pos
        assert phi(raw) > i / 17 and phi(raw) < (i + 1) / 17


# ------------------------------------------------------------------ nearest level

def test_nearest_level_equals_searchsorted_on_midpoints():
    """Independent formulation: count of exact FP64 midpoints strictly below rho."""
    q = O.nf4_codebook().astype(np.float64)
    mids = 0.5 * (q[:-1] + q[1:])
    rng = np.random.default_rng(0)
    rho = rng.uniform(-1, 1, 200000).astype(np.float32)
    # adversarial: the FP32 neighbours of every midpoint, and the midpoints themselves when exact
    adv = []
    for m in mids:
        f = np.float32(m)
        adv += [f, np.nextafter(f, np.float32(-2)), np.nextafter(f, np.float32(2))]
    rho = np.concatenate([rho, np.array(adv, dtype=np.float32), O.nf4_codebook()])
    ours = O.nearest_level(rho, O.nf4_codebook())
    theirs = np.searchsorted(mids, rho.astype(np.float64), side="left")  # ties -> lower index
    assert np.array_equal(ours, theirs.astype(np.uint8))


def test_nearest_level_tie_goes_low():
    q = O.nf4_codebook().astype(np.float64)
    for k in range(15):
        m = 0.5 * (q[k] + q[k + 1])
        if np.float64(np.float32(m)) == m:  # exact FP32 midpoint -> a true tie
            assert O.nearest_level(np.array([m], np.float32), O.nf4_codebook())[0] == k


@pytest.mark.parametrize("name", ["nf4", "int4", "fp4"])
def test_nearest_level_matches_midpoint_count_at_every_boundary(name):
    """Every codebook, at every midpoint's FP32 neighbours (two each side) and at the tiny
    values next to 0, inside [-1, 1]: the nearest level is the count of exact midpoints strictly below rho.
    The INT4 table has its midpoint at 0, where FP64 distances to the two levels tie for a
    subnormal rho; the sign of rho alone decides it (0 itself is a true tie, so it goes low)."""
    q = O.codebook(name).astype(np.float64)
    mids = 0.5 * (q[:-1] + q[1:])
    pts = [np.float32(0.0), np.float32(-0.0)]
    for m in np.concatenate([mids, [0.0]]):
        lo = hi = np.float32(m)
        pts.append(lo)
        for _ in range(2):
            lo, hi = np.nextafter(lo, np.float32(-2)), np.nextafter(hi, np.float32(2))
            pts += [lo, hi]
    rho = np.array(pts, dtype=np.float32)
    rho = rho[np.abs(rho) <= 1]  # |w / absmax| never exceeds 1
    ours = O.nearest_level(rho, O.codebook(name))
    theirs = np.searchsorted(mids, rho.astype(np.float64), side="left")
    assert np.array_equal(ours, theirs.astype(np.uint8))
    if name == "int4":
        tiny = np.array([1e-45, -1e-45, 0.0], np.float32)
        assert O.nearest_level(tiny, O.codebook(name)).tolist() == [8, 7, 7]


# ------------------------------------------------------------------ packing

def test_pack_roundtrip_and_layout():
    codes = np.arange(16, dtype=np.uint8).repeat(2)[:32]
    p = O.pack_codes(codes)
    assert p.size == 16
    # group of 8: byte i = e_i | e_{i+4} << 4
    e = codes[:8]
    assert list(p[:4]) == [int(e[i]) | (int(e[i + 4]) << 4) for i in range(4)]
    assert np.array_equal(O.unpack_codes(p), codes)


# ------------------------------------------------------------------ E4M3 and BF16

def test_e4m3_decode_matches_torch():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    ours = O.e4m3_value(codes)
    t = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(ours, t)
    assert O.e4m3_value(0x7E) == 448.0 and O.e4m3_value(0x01) == 2.0**-9 and O.e4m3_value(0x38) == 1.0


def test_e4m3_encode_matches_torch_everywhere_that_matters():
    vals = O.e4m3_value(np.arange(0, 0x7F)).astype(np.float64)
    mids = 0.5 * (vals[:-1] + vals[1:])
    pts = []
    for m in np.concatenate([vals, mids]):
        f = np.float32(m)
        pts += [f, np.nextafter(f, np.float32(0)), np.nextafter(f, np.float32(1e9))]
    rng = np.random.default_rng(1)
    pts = np.array(pts, dtype=np.float32)
    pts = np.concatenate([pts, -pts, rng.uniform(-448, 448, 100000).astype(np.float32),
                          (rng.standard_normal(20000) * 1e-3).astype(np.float32)])
    pts = pts[np.abs(pts) <= 448]
    ours = O.e4m3_encode(pts)
    theirs = torch.from_numpy(pts.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, theirs)


def test_e4m3_signed_zero():
    assert O.e4m3_encode(np.array([-1e-30], np.float32))[0] == 0x80
    assert O.e4m3_encode(np.array([1e-30], np.float32))[0] == 0x00


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 3,
                        np.array([1 + 2**-8, 1 + 3 * 2**-8, -(1 + 2**-8), 0.0, -0.0, 1e-40], np.float32)])
    ours = O.bf16_round_bits(x)
    theirs = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)


# ------------------------------------------------------------------ quantize / DQ

def _randW(n, k, seed=0, std=0.02):
    return (np.random.default_rng(seed).standard_normal((n, k)) * std).astype(np.float32)


def test_absmax_element_is_an_endpoint_and_decodes_to_scale():
    W = _randW(32, 256)
    q = O.quantize(W)
    blocks = W.reshape(-1, 64)
    idx = np.argmax(np.abs(blocks), axis=1)
    codes = q["codes"].reshape(-1, 64)
    picked = codes[np.arange(codes.shape[0]), idx]
    sgn = blocks[np.arange(blocks.shape[0]), idx] > 0
    assert np.all(picked == np.where(sgn, 15, 0))
    c1h = O.decode_scales(q["code8"], q["c2s"], q["mu"])
    what = O.bf16_bits_to_f32(O.dequantize_bf16_bits(q)).reshape(-1, 64)
    got = what[np.arange(what.shape[0]), idx]
    exp = O.bf16_bits_to_f32(O.bf16_round_bits(np.where(sgn, c1h, -c1h)))
    assert np.array_equal(got, exp)


def test_zero_stays_zero():
    W = _randW(8, 128, seed=3)
    W[0, 5] = 0.0
    W[3, 64:128] = 0.0  # an all-zero block
    q = O.quantize(W)
    assert q["codes"][0, 5] == 8 and np.all(q["codes"][3, 64:128] == 8)
    what = O.bf16_bits_to_f32(O.dequantize_bf16_bits(q))
    assert what[0, 5] == 0.0 and np.all(what[3, 64:128] == 0.0)
    assert q["c1"][3 * 2 + 1] == 0.0


def test_outlier_only_damages_its_own_block():
    W = _randW(16, 256, seed=4)
    a = O.quantize(W)
    W2 = W.copy()
    W2[5, 70] = 3.0  # block (5, 1)
    b = O.quantize(W2)
    ca, cb = a["codes"].reshape(-1, 64), b["codes"].reshape(-1, 64)
    changed = np.nonzero(np.any(ca != cb, axis=1))[0]
    assert list(changed) == [5 * 4 + 1]


def test_roundtrip_special_case_is_exact():
    """Every block holds +-c plus entries c*q_k (c a power of two): rho = q_k exactly,
    every c1 = c so mu = c, d = 0, c2s = 0, code8 = 0, c1_hat = c, and w_hat = bf16(W)."""
    q = O.nf4_codebook()
    rng = np.random.default_rng(5)
    c = np.float32(2.0**-6)
    k = rng.integers(0, 16, size=(64, 512)).astype(np.int64)
    k[:, ::64] = 15
    W = (q[k] * c).astype(np.float32)
    qq = O.quantize(W)
    assert np.array_equal(qq["codes"], k.astype(np.uint8))
    assert qq["mu"] == c and np.all(qq["c2s"] == 0) and np.all(qq["code8"] == 0)
    expected = torch.from_numpy(W).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.dequantize_bf16_bits(qq), expected)


def test_mean_is_exact_closed_form():
    """Block absmaxes j * 2^-10 for j = 1..n: the exact mean is (n+1)/2 * 2^-10."""
    n = 1024
    W = np.zeros((n, 64), np.float32)
    W[:, 0] = np.arange(1, n + 1, dtype=np.float32) * np.float32(2.0**-10)
    W[:, 1] = -0.5 * W[:, 0]
    q = O.quantize(W)
    assert q["mu"] == np.float32((n + 1) / 2 * 2.0**-10)


def test_double_quant_error_bound():
    W = _randW(256, 1024, seed=6)
    q = O.quantize(W)
    c1, mu = q["c1"].astype(np.float64), float(q["mu"])
    c1h = O.decode_scales(q["code8"], q["c2s"], q["mu"]).astype(np.float64)
    d = c1 - mu
    c2s = q["c2s"].astype(np.float64)[np.arange(c1.size) // 256]
    bound = np.abs(d) * 2.0**-4 + c2s * 2.0**-10 + 2.0**-23 * (np.abs(c1) + np.abs(d) + 1e-30)
    assert np.all(np.abs(c1h - c1) <= bound)
    # a group's largest |d| maps to +-448 exactly
    for g in range(q["c2s"].size):
        seg = np.abs(d[g * 256:(g + 1) * 256])
        j = g * 256 + int(np.argmax(seg))
        assert (q["code8"][j] & 0x7F) == 0x7E


def test_quantize_rejects_non_finite():
    W = _randW(4, 64)
    W[1, 3] = np.inf
    with pytest.raises(ValueError):
        O.quantize(W)


def test_brute_force_tiny_tensor_by_hand():
    """Recompute a tiny quantization with plain Python loops and floats."""
    W = _randW(2, 64, seed=7)
    q = O.quantize(W)
    table = [float(v) for v in O.nf4_codebook()]
    for r in range(2):
        c = max(abs(float(w)) for w in W[r])
        for j in range(64):
            rho = float(np.float32(W[r, j]) / np.float32(c))
            best = min(range(16), key=lambda k: (abs(rho - table[k]), k))
            assert q["codes"][r, j] == best


# ------------------------------------------------------------------ the pages' figures

def _page(fig_id):
    with open(os.path.join(GOLDEN, "page_figures.json")) as f:
        figs = {d["id"]: d for d in json.load(f)["figures"]}
    return figs[fig_id]


def _check(fig_id, value):
    d = _page(fig_id)
    assert round(value, d["digits"]) == pytest.approx(d["value"]), (fig_id, value, d)


def test_page_figures_bits_per_param():
    bpp = O.bits_per_param(4096, 4096)
    _check("bits_dq", bpp)
    _check("overhead_dq", bpp - 4.0)
    _check("overhead_first_level", O.bits_per_param(4096, 4096, double_quant=False) - 4.0)
    _check("bits_no_dq", O.bits_per_param(4096, 4096, double_quant=False))
    _check("saved_dq", O.bits_per_param(4096, 4096, double_quant=False) - bpp)


def test_page_figures_memory():
    bytes_per_param = O.bits_per_param(4096, 4096) / 8.0
    _check("base_8b_nf4dq_gb", 8.03e9 * bytes_per_param / GIB)
    _check("base_8b_bf16_gb", 8.03e9 * 2 / GIB)
    _check("base_14b_gb", 14e9 * 0.516 / GIB)
    shapes = [(4096, 4096), (1024, 4096), (1024, 4096), (4096, 4096), (14336, 4096), (14336, 4096), (4096, 14336)]
    n_adapter = 32 * sum(16 * (a + b) for a, b in shapes)
    _check("lora_8b_params", n_adapter)
    _check("lora_8b_w_grad_gb", n_adapter * 4 / GIB)
    _check("lora_8b_adamw_gb", n_adapter * 12 / GIB)
    _check("lora_4096_r16_params", 16 * (4096 + 4096))
    _check("lora_4096_r16_factor", 4096 * 4096 / (16 * 8192))
    _check("constants_65b_gb", (O.bits_per_param(4096, 4096, double_quant=False) - 4) * 65e9 / 8 / 1e9)
    _check("weights_65b_4bit_gb", 65e9 * 4 / 8 / 1e9)


# ------------------------------------------------------------------ forward / backward

def _case(M=6, N=24, K=128, r=4, seed=8):
    rng = np.random.default_rng(seed)
    What = rng.standard_normal((N, K))
    X = rng.standard_normal((M, K))
    A = rng.standard_normal((r, K)) / math.sqrt(K)
    B = rng.standard_normal((N, r)) * 0.1
    dY = rng.standard_normal((M, N))
    return What, X, A, B, dY


def test_fwd_bwd_match_torch_autograd():
    What, X, A, B, dY = _case()
    alpha, r = 8.0, 4
    Y, T = O.lora_fwd(What, X, A, B, alpha, r)
    dX, dA, dB = O.lora_bwd(What, X, dY, A, B, alpha, r)
    tW = torch.tensor(What)
    tX = torch.tensor(X, requires_grad=True)
    tA = torch.tensor(A, requires_grad=True)
    tB = torch.tensor(B, requires_grad=True)
    h = torch.nn.functional.linear(tX, tW) + (alpha / r) * torch.nn.functional.linear(torch.nn.functional.linear(tX, tA), tB)
    h.backward(torch.tensor(dY))
    assert np.allclose(Y, h.detach().numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(dX, tX.grad.numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(dA, tA.grad.numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(dB, tB.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_bwd_matches_finite_differences():
    What, X, A, B, dY = _case(M=3, N=8, K=64, r=2, seed=9)
    alpha, r = 4.0, 2
    L = lambda X_, A_, B_: float(np.sum(O.lora_fwd(What, X_, A_, B_, alpha, r)[0] * dY))
    dX, dA, dB = O.lora_bwd(What, X, dY, A, B, alpha, r)
    eps = 1e-6
    for arr, g in ((X, dX), (A, dA), (B, dB)):
        for idx in [(0, 0), (1, 1), (arr.shape[0] - 1, arr.shape[1] - 1)]:
            p, m = arr.copy(), arr.copy()
            p[idx] += eps
            m[idx] -= eps
            args_p = [p if arr is a else a for a in (X, A, B)]
            args_m = [m if arr is a else a for a in (X, A, B)]
            fd = (L(*args_p) - L(*args_m)) / (2 * eps)
            assert fd == pytest.approx(g[idx], rel=1e-6, abs=1e-8)


def test_fwd_one_hot_inputs_pick_columns():
    """X = e_j rows pick column j of W_hat; with W_hat = 0 and one-hot adapters the LoRA
    term is alpha/r * B[n, a] * A[a, j]: catches a transposed operand or a wrong scale."""
    N, K, r = 5, 64, 3
    rng = np.random.default_rng(10)
    What = rng.standard_normal((N, K))
    X = np.zeros((2, K)); X[0, 7] = 1; X[1, 40] = 1
    A = np.zeros((r, K)); B = np.zeros((N, r))
    Y, _ = O.lora_fwd(What, X, A, B, 6.0, r)
    assert np.array_equal(Y[0], What[:, 7]) and np.array_equal(Y[1], What[:, 40])
    A[1, 40] = 1.0; B[3, 1] = 1.0
    Y, _ = O.lora_fwd(np.zeros((N, K)), X, A, B, 6.0, r)
    exp = np.zeros((2, N)); exp[1, 3] = 2.0
    assert np.array_equal(Y, exp)


def test_special_cases_alpha_zero_and_B_zero():
    What, X, A, B, dY = _case(seed=11)
    Y0, _ = O.lora_fwd(What, X, A, B, 0.0, 4)
    assert np.allclose(Y0, X @ What.T)
    dX, dA, dB = O.lora_bwd(What, X, dY, A, np.zeros_like(B), 8.0, 4)
    assert np.all(dA == 0) and np.allclose(dX, dY @ What)


# ------------------------------------------------------------------ merge / export

from fractions import Fraction


def _bf16_nearest_by_enumeration(x: float) -> int:
    """BF16 bit pattern nearest to the float64 x (ties to the even pattern), by exact
    rational distances to the neighbouring patterns -- no rounding mode involved."""
    sign = 0x8000 if math.copysign(1.0, x) < 0 else 0
    a = abs(x)
    t = int(np.array(a, np.float32).view(np.uint32)) >> 16  # near a (within a few patterns)
    best, best_d = None, None
    for cand in range(max(t - 2, 0), t + 3):
        v = Fraction(float(np.array(cand << 16, np.uint32).view(np.float32)))
        d = abs(Fraction(a) - v)
        if best is None or d < best_d or (d == best_d and cand % 2 == 0):
            best, best_d = cand, d
    return best | sign


def test_bf16_round_f64_is_one_correct_rounding():
    rng = np.random.default_rng(20)
    vals = list(rng.standard_normal(400) * 10.0 ** rng.integers(-6, 4, 400))
    # exact BF16 midpoints and points a hair off them (where a double rounding goes wrong)
    for b in rng.integers(0x3000, 0x4800, 100):
        lo = float(np.array(int(b) << 16, np.uint32).view(np.float32))
        hi = float(np.array((int(b) + 1) << 16, np.uint32).view(np.float32))
        mid = (lo + hi) / 2
        vals += [mid, -mid, mid + abs(mid) * 2.0**-40, mid - abs(mid) * 2.0**-40, mid * (1 + 2.0**-30)]
    vals += [0.0, 3.0e-40, -7.1e-39, 1.0 + 2.0**-8 + 2.0**-40]
    x = np.array(vals, np.float64)
    got = O.bf16_round_f64_bits(x)
    exp = np.array([_bf16_nearest_by_enumeration(v) for v in vals], np.uint16)
    assert np.array_equal(got, exp)


def test_merge_is_the_forward_through_one_matrix():
    """X W'^T equals the adapted forward of X for every X (before W' is rounded): a
    transposed, unscaled or sign-flipped adapter fails.  Non-square, r > 1."""
    W = _randW(48, 192, seed=21)
    q = O.quantize(W)
    rng = np.random.default_rng(22)
    r, alpha = 5, 11.0
    A = rng.standard_normal((r, 192))
    B = rng.standard_normal((48, r))
    X = rng.standard_normal((7, 192))
    _, exact = O.merge(q, A, B, alpha, r)
    Y, _ = O.lora_fwd(O.dequantize_f64(q), X, A, B, alpha, r)
    assert np.allclose(X @ exact.T, Y, rtol=1e-12, atol=1e-12)


def test_merge_special_cases():
    W = _randW(32, 128, seed=23)
    q = O.quantize(W)
    A = np.zeros((3, 128))
    B = np.zeros((32, 3))
    bits, _ = O.merge(q, A, B, 6.0, 3)
    assert np.array_equal(bits, O.dequantize_bf16_bits(q))  # B = 0: the dequantized base
    A[2, 70] = 1.0
    B[9, 2] = 1.0
    bits, _ = O.merge(q, A, B, 6.0, 3)  # one-hot adapter: only (9, 70) moves, by alpha/r
    base = O.dequantize_bf16_bits(q)
    diff = np.argwhere(bits != base)
    assert [tuple(d) for d in diff] == [(9, 70)]
    w = float(O.bf16_bits_to_f32(base[9, 70]))
    assert int(bits[9, 70]) == _bf16_nearest_by_enumeration(w + 2.0)


def test_requantize_unchanged_special_weight_restores_codes():
    """NF4 codes -> BF16 merge with B = 0 -> quantize again: with block absmaxes +-c exact,
    the re-quantized codes and constants equal the originals."""
    qt = O.nf4_codebook()
    rng = np.random.default_rng(24)
    c = np.float32(2.0**-5)
    k = rng.integers(0, 16, size=(32, 256)).astype(np.int64)
    k[:, ::64] = 0
    W = (qt[k] * c).astype(np.float32)
    q = O.quantize(W)
    bits, _ = O.merge(q, np.zeros((2, 256)), np.zeros((32, 2)), 4.0, 2)
    q2 = O.quantize_bf16(bits)
    assert np.array_equal(q2["codes"], q["codes"]) and np.array_equal(q2["codes"], k.astype(np.uint8))
    assert q2["mu"] == c and np.array_equal(q2["code8"], q["code8"]) and np.array_equal(q2["c2s"], q["c2s"])


# ------------------------------------------------------------------ adapter optimizer step

def _bf16_bits(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("step,wd", [(1, 0.0), (7, 0.01), (1000, 0.1)])
def test_adamw_matches_torch_adamw(step, wd):
    """One step from a given state equals torch.optim.AdamW in float64 (a separate
    implementation of the same published update)."""
    rng = np.random.default_rng(30 + step)
    n = 999
    master = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    v = (rng.random(n) * 1e-6).astype(np.float32)
    g = _bf16_bits(rng.standard_normal(n) * 1e-3)
    lr, b1, b2, eps = 2e-4, 0.9, 0.999, 1e-8
    th32, m32, v32, pbits, th = O.adamw_step(master, m, v, g, step, lr, b1, b2, eps, wd)
    p = torch.tensor(master.astype(np.float64), requires_grad=True)
    opt = torch.optim.AdamW([p], lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd, foreach=False)
    opt.state[p] = {"step": torch.tensor(float(step - 1), dtype=torch.float64),
                    "exp_avg": torch.tensor(m.astype(np.float64)), "exp_avg_sq": torch.tensor(v.astype(np.float64))}
    p.grad = torch.tensor(O.bf16_bits_to_f32(g).astype(np.float64))
    opt.step()
    assert np.allclose(th, p.detach().numpy(), rtol=1e-12, atol=1e-18)
    assert np.allclose(m32, opt.state[p]["exp_avg"].numpy(), rtol=1e-6, atol=0)
    assert np.allclose(v32, opt.state[p]["exp_avg_sq"].numpy(), rtol=1e-6, atol=0)
    assert np.array_equal(pbits, _bf16_bits(th32))


def test_adamw_constant_gradient_closed_form():
    """With a constant gradient c, no decay and zero initial moments, the bias-corrected
    moments are exactly c and c^2, so every step moves theta by lr |c| / (|c| + eps)
    against the sign of c."""
    n = 64
    rng = np.random.default_rng(40)
    c = rng.choice([-1.0, 1.0], n) * 2.0 ** rng.integers(-12, -4, n)
    g = _bf16_bits(c)
    th0 = (rng.standard_normal(n) * 0.05).astype(np.float32)
    th, m, v = th0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    lr, eps = 1e-3, 1e-8
    for t in range(1, 6):
        th, m, v, _, _ = O.adamw_step(th, m, v, g, t, lr, 0.9, 0.999, eps, 0.0)
    exp = th0.astype(np.float64) - 5 * lr * np.sign(c) * np.abs(c) / (np.abs(c) + eps)
    assert np.allclose(th, exp, rtol=0, atol=2e-7 * 5 * lr + 5 * 2.0**-24 * np.abs(exp))


def test_adamw_pure_decay():
    n = 32
    th0 = np.linspace(-1, 1, n).astype(np.float32)
    th, m, v = th0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    g = np.zeros(n, np.uint16)
    for t in range(1, 4):
        th, m, v, _, _ = O.adamw_step(th, m, v, g, t, 0.01, 0.9, 0.999, 1e-8, 0.5)
    assert np.all(m == 0) and np.all(v == 0)
    assert np.allclose(th, th0.astype(np.float64) * (1 - 0.005) ** 3, rtol=1e-6)


# ------------------------------------------------------------------ format variants

def test_variant_codebooks_closed_forms():
    """INT4: 16 evenly spaced levels -1 + 2i/15; FP4: the E2M1 magnitudes over 6, with the
    duplicated top level never chosen first."""
    q = O.codebook("int4").astype(np.float64)
    exact = np.array([-1 + 2 * i / 15 for i in range(16)])
    assert np.all(np.abs(q - exact) <= 2.0**-24) and q[0] == -1 and q[15] == 1 and not np.any(q == 0)
    f = O.codebook("fp4").astype(np.float64)
    e2m1 = sorted({s * m for s in (-1, 1) for m in (0, 0.5, 1, 1.5, 2, 3, 4, 6)})
    assert np.all(np.abs(f[:15] * 6 - np.array(e2m1)) <= 6 * 2.0**-24) and f[15] == f[14] == 1
    assert np.all(np.diff(f[:15]) > 0)
    # nearest-level assignment never picks the duplicate
    assert np.all(O.nearest_level(np.linspace(-1, 1, 4001, dtype=np.float32), O.codebook("fp4")) <= 14)


def test_e5m2_matches_torch():
    codes = np.arange(0, 0x7C)
    assert np.array_equal(O.e5m2_value(codes).astype(np.float32),
                          torch.from_numpy(codes.astype(np.uint8)).view(torch.float8_e5m2).float().numpy())
    vals = O.e5m2_value(codes)
    mids = 0.5 * (vals[:-1] + vals[1:])
    pts = []
    for m in np.concatenate([vals, mids]):
        f = np.float32(m)
        pts += [f, np.nextafter(f, np.float32(0)), np.nextafter(f, np.float32(1e9))]
    pts = np.array(pts, np.float32)
    pts = np.concatenate([pts, -pts, np.random.default_rng(41).uniform(-57344, 57344, 20000).astype(np.float32)])
    pts = pts[np.abs(pts) <= 57344]
    ref = torch.from_numpy(pts).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(O.e5m2_encode(pts), ref)


def test_int8_encode_rounding_by_hand():
    s = np.array([0.5, 1.5, 2.5, -0.5, -1.5, 126.5, 127.0, -127.0, 3.49999976, -0.0], np.float32)
    assert list(O.int8_encode(s).view(np.int8)) == [0, 2, 2, 0, -2, 126, 127, -127, 3, 0]


@pytest.mark.parametrize("dq,rel", [("e4m3", 2.0**-4), ("e5m2", 2.0**-3), ("int8", 0.0), ("none", 0.0)])
def test_variant_double_quant_error_bounds(dq, rel):
    """|c1 - c1_hat| <= |d| * 2^-(m+1) + c2s * (half a step at the bottom of the format),
    plus FP32 rounding; exact without double quantization.  INT8 steps are c2s wide."""
    W = _randW(256, 1024, seed=42)
    q = O.quantize(W, dq=dq)
    c1 = q["c1"].astype(np.float64)
    c1h = O.decode_scales(q["code8"], q["c2s"], q["mu"], dq).astype(np.float64)
    if dq == "none":
        assert np.array_equal(c1h, c1)
        return
    d = c1 - float(q["mu"])
    c2s = q["c2s"].astype(np.float64)[np.arange(c1.size) // 256]
    floor = {"e4m3": 2.0**-10, "e5m2": 2.0**-17, "int8": 0.5}[dq]
    bound = np.abs(d) * rel + c2s * floor + 2.0**-22 * (np.abs(c1) + np.abs(d))
    assert np.all(np.abs(c1h - c1) <= bound)


def test_nf4_reconstructs_gaussian_weights_best():
    """The pages' claim ([4-Bit] Sec. 2 "1. 4-bit NormalFloat"; [65B] "NF4"): at the same 4
    bits, NF4 levels reconstruct normally distributed weights better than evenly spaced
    INT4 or FP4 levels.  Checked with and without double quantization."""
    W = _randW(512, 1024, seed=43)
    for dq in ("e4m3", "none"):
        mse = {cb: float(np.mean((O.dequantize_f64(O.quantize(W, codebook_name=cb, dq=dq)) - W.astype(np.float64)) ** 2))
               for cb in O.CODEBOOKS}
        assert mse["nf4"] < mse["int4"] and mse["nf4"] < mse["fp4"], (dq, mse)


def test_variant_storage_bits():
    """8-bit second-level formats keep the 4.127 bits/param; without double quantization the
    constants cost 32/64 = 0.5 bits/param ([4-Bit] Sec. 2: 0.500 bits per parameter)."""
    for dq in ("e4m3", "e5m2", "int8"):
        sz = O.quant_sizes(4096, 4096, dq)
        assert 8 * sum(sz.values()) / 4096**2 == pytest.approx(4.127, abs=5e-4)
    sz = O.quant_sizes(4096, 4096, "none")
    assert 8 * sum(sz.values()) / 4096**2 == 4.5


def test_variant_zero_block_and_exact_special_case():
    """An all-zero block takes the level nearest 0 (code 8 for NF4, 7 for FP4's zero and for
    INT4, whose two middle levels tie); with power-of-two constants and every weight a level
    times that constant, every format reproduces bf16(W) exactly without double
    quantization."""
    W = np.zeros((2, 64), np.float32)
    assert np.all(O.quantize(W, codebook_name="int4", dq="none")["codes"] == 7)
    assert np.all(O.quantize(W, codebook_name="fp4", dq="none")["codes"] == 7)
    assert np.all(O.quantize(W)["codes"] == 8)
    rng = np.random.default_rng(44)
    for cb in O.CODEBOOKS:
        t = O.codebook(cb)
        k = rng.integers(0, 15, size=(16, 256))
        k[:, ::64] = 0
        W = (t[k] * np.float32(2.0**-6)).astype(np.float32)
        q = O.quantize(W, codebook_name=cb, dq="none")
        assert np.array_equal(t[q["codes"]], t[k])
        exp = torch.from_numpy(W).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(O.dequantize_bf16_bits(q), exp)


# ---------------------------------------------------------------- MLP block


def test_silu_closed_forms():
    """silu(0) = 0, slope 1/2 at 0, silu(x) - silu(-x) = x, silu -> x for large x and -> 0 for
    very negative x, and the value at 1 is 1 / (1 + 1/e)."""
    x = np.linspace(-30.0, 30.0, 241)
    assert O.silu(0.0) == 0.0
    assert np.allclose(O.silu(x) - O.silu(-x), x, rtol=0, atol=1e-12)
    h = 1e-6
    assert (O.silu(h) - O.silu(-h)) / (2 * h) == pytest.approx(0.5, rel=1e-9)
    assert O.silu(40.0) == pytest.approx(40.0, rel=1e-15)
    assert abs(O.silu(-40.0)) < 1e-15
    assert O.silu(1.0) == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), rel=1e-15)
    assert np.allclose(O.silu(x), torch.nn.functional.silu(torch.tensor(x)).numpy(), rtol=1e-14, atol=1e-14)


def _mlp_case(M=3, d=8, f=16, r=2, seed=21):
    rng = np.random.default_rng(seed)
    Wg = rng.standard_normal((f, d)) * 0.3
    Wu = rng.standard_normal((f, d)) * 0.3
    Wd = rng.standard_normal((d, f)) * 0.3
    X = rng.standard_normal((M, d))
    As = [rng.standard_normal((r, d)) * 0.3, rng.standard_normal((r, d)) * 0.3, rng.standard_normal((r, f)) * 0.3]
    Bs = [rng.standard_normal((f, r)) * 0.2, rng.standard_normal((f, r)) * 0.2, rng.standard_normal((d, r)) * 0.2]
    dY = rng.standard_normal((M, d))
    return Wg, Wu, Wd, X, As, Bs, dY


def test_mlp_bwd_matches_finite_differences():
    """Every gradient of the MLP block against central differences of the scalar loss
    sum(dY * Y): a dropped term, a wrong sign or a swapped operand in the chain fails."""
    Wg, Wu, Wd, X, As, Bs, dY = _mlp_case()
    alpha, r = 6.0, 2

    def loss(X_, As_, Bs_):
        return float(np.sum(O.mlp_fwd(Wg, Wu, Wd, X_, As_, Bs_, alpha, r)[0] * dY))

    dX, dAs, dBs = O.mlp_bwd(Wg, Wu, Wd, X, dY, As, Bs, alpha, r)
    eps = 1e-6
    targets = [("X", None, X, dX)] + [("A", i, As[i], dAs[i]) for i in range(3)] + [("B", i, Bs[i], dBs[i]) for i in range(3)]
    for kind, i, arr, grad in targets:
        for idx in [(0, 0), (arr.shape[0] - 1, arr.shape[1] - 1), (arr.shape[0] // 2, 1)]:
            def perturbed(delta):
                a = arr.copy()
                a[idx] += delta
                Xp = a if kind == "X" else X
                Ap = [a if (kind == "A" and j == i) else As[j] for j in range(3)]
                Bp = [a if (kind == "B" and j == i) else Bs[j] for j in range(3)]
                return loss(Xp, Ap, Bp)
            fd = (perturbed(eps) - perturbed(-eps)) / (2 * eps)
            assert fd == pytest.approx(grad[idx], rel=1e-5, abs=1e-8), (kind, i, idx)


def test_mlp_matches_torch_autograd():
    """The same block written with torch's own silu and autograd gives the same outputs and
    gradients."""
    Wg, Wu, Wd, X, As, Bs, dY = _mlp_case(M=4, d=16, f=24, r=3, seed=5)
    alpha, r = 9.0, 3
    Y, G, U, H = O.mlp_fwd(Wg, Wu, Wd, X, As, Bs, alpha, r)
    dX, dAs, dBs = O.mlp_bwd(Wg, Wu, Wd, X, dY, As, Bs, alpha, r)
    F = torch.nn.functional
    tX = torch.tensor(X, requires_grad=True)
    tA = [torch.tensor(a, requires_grad=True) for a in As]
    tB = [torch.tensor(b, requires_grad=True) for b in Bs]
    s = alpha / r

    def lin(W, x, A, B):
        return F.linear(x, torch.tensor(W)) + s * F.linear(F.linear(x, A), B)

    tY = lin(Wd, F.silu(lin(Wg, tX, tA[0], tB[0])) * lin(Wu, tX, tA[1], tB[1]), tA[2], tB[2])
    tY.backward(torch.tensor(dY))
    assert np.allclose(Y, tY.detach().numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(dX, tX.grad.numpy(), rtol=1e-11, atol=1e-12)
    for i in range(3):
        assert np.allclose(dAs[i], tA[i].grad.numpy(), rtol=1e-11, atol=1e-12)
        assert np.allclose(dBs[i], tB[i].grad.numpy(), rtol=1e-11, atol=1e-12)


def test_mlp_special_cases():
    """With the up projection zero (weights and B), U = 0, so H = 0 and Y = 0, and no gradient
    reaches the gate's adapter; with the gate projection zero, G = 0 and H = silu(0) U = 0."""
    Wg, Wu, Wd, X, As, Bs, dY = _mlp_case(seed=3)
    alpha, r = 4.0, 2
    Bz = [Bs[0], np.zeros_like(Bs[1]), Bs[2]]
    Y, G, U, H = O.mlp_fwd(Wg, np.zeros_like(Wu), Wd, X, As, Bz, alpha, r)
    assert np.all(U == 0) and np.all(H == 0) and np.all(Y == 0)
    dX, dAs, dBs = O.mlp_bwd(Wg, np.zeros_like(Wu), Wd, X, dY, As, Bz, alpha, r)
    assert np.all(dAs[0] == 0) and np.all(dBs[0] == 0)
    Bg = [np.zeros_like(Bs[0]), Bs[1], Bs[2]]
    _, G0, _, H0 = O.mlp_fwd(np.zeros_like(Wg), Wu, Wd, X, As, Bg, alpha, r)
    assert np.all(G0 == 0) and np.all(H0 == 0)

