"""GPU parity at the edges the random-data tests do not reach.

- The nearest-level decision ("QLoRA -- Fine-Tuning a 65B Model on One GPU", "Quantization in
  one paragraph": each weight is stored as the index of the nearest level).  The device picks
  the code by counting thresholds below rho; these cases put rho exactly on every midpoint
  between adjacent levels, on the FP32 values around it and around every level, for both
  signs and every first-level codebook, and compare the codes with the oracle's brute force.
- Config 5 at layer 0 (the 70B-class gate projection, 28672 x 8192): every code, constant
  and decoded weight against the oracle, not a sample.
- The fused mid-size GEMMs (16 < M < 1024) at layer shapes: 4096 x 4096 at M = 512 and
  14336 x 4096 at M = 256, forward and backward in full.
"""

import numpy as np
import pytest
import torch

import oracle as O
from bit_nf4_quantized_dq_amd import inputs as I

pytestmark = pytest.mark.gpu
TOL = 1e-2


def _np(t):
    return t.detach().cpu().numpy()


def _f64(t_bf16):
    return t_bf16.detach().float().cpu().numpy().astype(np.float64)


def normwise(got, ref):
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(got - ref)) / (den if den > 0 else 1.0))


def _f32_neighbours(x, n):
    """The FP32 values x, and n steps below and above it."""
    out = [np.float32(x)]
    lo = hi = np.float32(x)
    for _ in range(n):
        lo = np.nextafter(lo, np.float32(-np.inf))
        hi = np.nextafter(hi, np.float32(np.inf))
        out += [lo, hi]
    return out


def _decision_points(table):
    """FP32 values of rho at and around every decision boundary of `table`: for each pair of
    adjacent levels, the exact midpoint (FP64, exact for FP32 operands) rounded down and up
    to FP32 with two neighbours each side, and each level with one neighbour each side.
    Only points inside [-1, 1] are kept (|rho| <= 1 in a block with absmax 1)."""
    t = table.astype(np.float64)
    pts = []
    for k in range(15):
        mid = 0.5 * (t[k] + t[k + 1])
        f = np.float32(mid)
        down = f if float(f) <= mid else np.nextafter(f, np.float32(-np.inf))
        up = f if float(f) >= mid else np.nextafter(f, np.float32(np.inf))
        pts += _f32_neighbours(down, 2) + _f32_neighbours(up, 2)
    for v in table:
        pts += _f32_neighbours(v, 1)
    pts = np.array(pts, dtype=np.float32)
    pts = np.concatenate([pts, -pts])
    return np.unique(pts[np.abs(pts) <= 1.0])


def _assert_straddles(table):
    """The points around each midpoint between distinct adjacent levels reach both levels'
    codes (checks the construction above, not the device)."""
    t = table.astype(np.float64)
    for k in range(15):
        if t[k] == t[k + 1]:
            continue
        mid = 0.5 * (t[k] + t[k + 1])
        near = np.array([p for p in _decision_points(table) if abs(float(p) - mid) <= 4e-7 * max(abs(mid), 1e-3)],
                        np.float32)
        assert set(O.nearest_level(near, table).tolist()) == {k, k + 1}, (k, mid)


def _boundary_weight(pts, scale, rows_per_case=16, d_in=256):
    """Blocks of 64 whose first entry is +-scale (so c1 = scale) and whose other 63 entries are
    scale * p for the decision points p, cycled.  With scale a power of two, rho = p exactly;
    otherwise rho is fl32(fl32(scale * p) / scale), which lands within an ulp of p."""
    n_blocks = rows_per_case * d_in // 64
    body = np.resize(pts, (n_blocks, 63)).astype(np.float32)
    W = np.empty((n_blocks, 64), np.float32)
    W[:, 1:] = (body * np.float32(scale)).astype(np.float32)
    W[:, 0] = np.where(np.arange(n_blocks) % 2 == 0, np.float32(scale), np.float32(-scale))
    return W.reshape(rows_per_case, d_in)


@pytest.mark.parametrize("cb", ["nf4", "int4", "fp4"])
def test_nearest_level_at_decision_boundaries(gpu_lib, cb):
    from bit_nf4_quantized_dq_amd import dequantize, quantize

    table = O.codebook(cb)
    pts = _decision_points(table)
    # scales: 1 (rho = w), 2^-7 (rho = w / c exactly), 0.37 (rho off the grid by the division)
    W = np.concatenate([_boundary_weight(pts, s) for s in (1.0, 2.0**-7, 0.37)], axis=0)
    W = np.concatenate([W, np.roll(W, 7, axis=1)], axis=0)  # each point in another lane position
    oq = O.quantize(W, codebook_name=cb)
    _assert_straddles(table)
    q = quantize(torch.from_numpy(W).cuda(), codebook=cb)
    torch.cuda.synchronize()
    got = _np(q.codes).reshape(-1)
    exp = oq["packed"].reshape(-1)
    bad = np.nonzero(got != exp)[0]
    assert bad.size == 0, f"{cb}: {bad.size} code bytes differ, first at byte {bad[:4]}"
    assert np.array_equal(_np(q.code8), oq["code8"])
    w = dequantize(q)
    assert np.array_equal(_np(w.view(torch.int16)).view(np.uint16), O.dequantize_bf16_bits(oq))


def test_nearest_level_at_decision_boundaries_many_scales(gpu_lib):
    """rho = fl32(w / c1) for many block constants c1: each block holds +-c1 and the FP32
    values fl32(c1 p) and one ulp either side of it for the decision points p, so that the
    rounded quotient lands on and around every boundary.  The constants span 2^-40 .. 2^100
    (the range where the device forms the quotient from a reciprocal, exactly) and the FP32
    values just outside it at both ends (the correctly rounded division)."""
    from bit_nf4_quantized_dq_amd import quantize

    table = O.nf4_codebook()
    pts = _decision_points(table)
    rng = np.random.default_rng(11)
    scales = [np.float32(m * 2.0**e) for m, e in zip(rng.uniform(1, 2, 48), rng.integers(-39, 99, 48))]
    scales += [np.float32(s) for s in rng.uniform(0.005, 0.2, 12)]
    lo, hi = np.float32(2.0**-40), np.float32(2.0**100)
    scales += [lo, np.nextafter(lo, np.float32(0)), np.nextafter(lo, np.float32(np.inf)),
               hi, np.nextafter(hi, np.float32(np.inf)), np.nextafter(hi, np.float32(0))]
    blocks = []
    for sc in scales:
        w = (pts.astype(np.float32) * sc).astype(np.float32)
        w = np.concatenate([np.nextafter(w, np.float32(-np.inf)), w, np.nextafter(w, np.float32(np.inf))])
        w = np.clip(w, -sc, sc).astype(np.float32)
        nb = -(-w.size // 63)
        body = np.resize(w, (nb, 63))
        b = np.empty((nb, 64), np.float32)
        b[:, 1:] = body
        b[:, 0] = np.where(np.arange(nb) % 2 == 0, sc, -sc)
        blocks.append(b)
    B = np.concatenate(blocks, axis=0)
    B = np.resize(B, (-(-B.shape[0] // 64) * 64, 64))  # whole rows of 256, rows a multiple of 16
    W = B.reshape(-1, 256)
    oq = O.quantize(W)
    q = quantize(torch.from_numpy(W).cuda())
    torch.cuda.synchronize()
    got = _np(q.codes).reshape(-1)
    exp = oq["packed"].reshape(-1)
    bad = np.nonzero(got != exp)[0]
    assert bad.size == 0, f"{bad.size} code bytes differ, first at byte {bad[:4]}"
    assert np.array_equal(_np(q.code8), oq["code8"])


def test_nearest_level_at_decision_boundaries_bf16_input(gpu_lib):
    """BF16 weights: the BF16 values next to each NF4 midpoint (a BF16 rho has 8 significant
    bits, so the boundary is straddled by its two BF16 neighbours)."""
    from bit_nf4_quantized_dq_amd import quantize_bf16

    t = O.nf4_codebook().astype(np.float64)
    pts = []
    for k in range(15):
        mid = 0.5 * (t[k] + t[k + 1])
        b = O.bf16_round_f64_bits(np.array([mid]))[0]
        for d in (-2, -1, 0, 1, 2):
            pts.append(O.bf16_bits_to_f32(np.array([(int(b) + d) & 0xFFFF], np.uint16))[0])
    pts = np.array(pts, np.float32)
    pts = np.concatenate([pts, -pts])
    pts = pts[np.abs(pts) <= 1.0]
    W = _boundary_weight(pts, 1.0)
    Wb = O.bf16_round_bits(W)  # exact: every entry is a BF16 value already
    assert np.array_equal(O.bf16_bits_to_f32(Wb), W)
    oq = O.quantize_bf16(Wb)
    q = quantize_bf16(torch.from_numpy(Wb.view(np.int16)).view(torch.bfloat16).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(_np(q.codes).reshape(-1), oq["packed"].reshape(-1))


@pytest.mark.timeout(900)
def test_config5_layer0_gate_full(gpu_lib):
    """70B-class gate projection, layer 0 (28672 x 8192, 235M weights): packed codes, code8,
    c2s, mu and every decoded weight against the oracle."""
    from bit_nf4_quantized_dq_amd import dequantize, quantize

    idx, layer = 4, 0
    shp = I.SEVENTY_B_LAYER[idx]
    print(f"70B layer {layer} {shp.name} {shp.d_out}x{shp.d_in}: quantize on the GPU", flush=True)
    W = I.weight(5, idx, shp.d_out, shp.d_in, 0.015, layer)
    q = quantize(W.cuda())
    w = dequantize(q)
    torch.cuda.synchronize()
    got_codes = _np(q.codes)
    got_c8, got_c2s, got_mu = _np(q.code8), _np(q.c2s), _np(q.mu)
    got_w = _np(w.view(torch.int16)).view(np.uint16).reshape(-1)
    del w, q
    torch.cuda.empty_cache()
    print("oracle quantize", flush=True)
    oq = O.quantize(W.numpy())
    del W
    assert np.array_equal(got_codes, oq["packed"].reshape(-1)), "packed codes"
    assert np.array_equal(got_c8, oq["code8"]), "code8"
    assert np.array_equal(got_c2s.view(np.uint32), oq["c2s"].view(np.uint32)), "c2s"
    assert got_mu.view(np.uint32)[0] == np.float32(oq["mu"]).view(np.uint32), "mu"
    print("oracle dequantize", flush=True)
    assert np.array_equal(got_w, O.dequantize_bf16_bits(oq).reshape(-1)), "decoded weights"


MID_CASES = [
    # cfg, idx, d_out, d_in, M: the fused per-tile decode GEMMs at layer shapes
    (3, 5, 4096, 4096, 512),
    (4, 4, 14336, 4096, 256),
]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("cfg,idx,N,K,M", MID_CASES)
def test_fused_mid_m_gemms_at_layer_shapes(gpu_lib, cfg, idx, N, K, M):
    from bit_nf4_quantized_dq_amd import linear_bwd, linear_fwd, quantize

    r, alpha = 16, 32.0
    print(f"fused mid-M {N}x{K} M={M}", flush=True)
    c = I.linear_case(cfg, idx, N, K, M, r, 0.02)
    q = quantize(c["W"].cuda())
    X, A, Bm, dY = (c[k].cuda() for k in ("X", "A", "B", "dY"))
    T = torch.empty(M, r, dtype=torch.bfloat16, device="cuda")
    Y = linear_fwd(q, X, A, Bm, alpha, T_save=T)
    dX, dA, dB = linear_bwd(q, X, dY, A, Bm, alpha, T_saved=T)
    torch.cuda.synchronize()
    oq = O.quantize(c["W"].numpy())
    assert np.array_equal(_np(q.codes), oq["packed"].reshape(-1))
    what = O.dequantize_f64(oq)
    Xf, Af, Bf, dYf = (_f64(c[k]) for k in ("X", "A", "B", "dY"))
    Yr, Tr = O.lora_fwd(what, Xf, Af, Bf, alpha, r)
    dXr, dAr, dBr = O.lora_bwd(what, Xf, dYf, Af, Bf, alpha, r)
    for name, got, ref in (("Y", Y, Yr), ("T", T, Tr), ("dX", dX, dXr), ("dA", dA, dAr), ("dB", dB, dBr)):
        e = normwise(_f64(got), ref)
        assert e <= TOL, (name, e)
