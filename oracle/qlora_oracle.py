"""Plain CPU oracle: NF4 codebook, blockwise absmax quantization, double quantization of
the block constants, dequantization, and the LoRA-augmented forward/backward.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  FP64 math unless a step is
defined in FP32; FP32 steps use NumPy float32 scalars/arrays, whose +, -, *, / are
IEEE round-to-nearest-even and never fused.

Sources (cited by page title and section):
  [4-Bit]  "QLoRA: Quantize Base Weights to 4-Bit" -- Section 2 ("1. 4-bit NormalFloat",
           "2. Double Quantization"), Section 3 (the dequantize-compute loop).
  [65B]    "QLoRA -- Fine-Tuning a 65B Model on One GPU" -- "Prerequisite: LoRA's low-rank
           update", "Quantization in one paragraph", "NF4: sixteen levels shaped like the
           weights", "Double quantization: the constants are not free", "Where the
           gradients actually go".
  [Consumer] "What is 4-bit NormalFloat (NF4) quantization and why is it
           information-theoretically optimal?" -- FAQ on double quantization.
"""

from __future__ import annotations

import math
from fractions import Fraction

import mpmath
import numpy as np

BLOCK1 = 64  # weights per first-level absmax block ([4-Bit] Sec. 2 "2. Double Quantization")
BLOCK2 = 256  # first-level constants per second-level group (same passage)
E4M3_MAX = 448.0  # largest finite OCP FP8 E4M3 value (S.1111.110 = 1.75 * 2^8)

# --------------------------------------------------------------------------------------
# NF4 codebook
# --------------------------------------------------------------------------------------


def _q_normal(num: int, den: int) -> mpmath.mpf:
    """Standard-normal quantile Q(num/den) at 60 significant digits.

    Evaluated on the lower half only and mirrored, so Q(1-p) == -Q(p) holds exactly
    (reading R(1)): the interior of the table is then exactly antisymmetric."""
    with mpmath.workdps(60):
        if 2 * num > den:
            return -_q_normal(den - num, den)
        p = mpmath.mpf(num) / den
        return mpmath.sqrt(2) * mpmath.erfinv(2 * p - 1)


def nf4_codebook_exact() -> list:
    """The 16 NF4 levels as 60-digit mpmath numbers, before FP32 rounding.

    [4-Bit] Sec. 2 "1. 4-bit NormalFloat": q_i = 1/2 (Q(i/(2^k+1)) + Q((i+1)/(2^k+1))),
    k = 4, Q the standard-normal quantile function; 0 is represented exactly and q_15 is
    finite.  [65B] "NF4": 8 negative and 8 non-negative levels including a true 0, and the
    endpoints are exactly -1 and +1 so a block's absmax survives.

    Reading R (the printed formula gives q_0 = -inf, since Q(0) = -inf):
      (1) levels 1..15 follow the formula literally (q_8 = 0 exactly);
      (2) the tail level q_0, whose bin [0, 1/17] has one infinite edge, takes the
          quantile at the bin's probability midpoint, Q(1/34);
      (3) each side is scaled by its own extreme: negatives by |q_0|, non-negatives by
          q_15, so the endpoints are exactly -1 and +1 and 0 stays 0.
    """
    den = 2**4 + 1  # 17
    raw = [None] * 16
    with mpmath.workdps(60):
        raw[0] = _q_normal(1, 2 * den)  # Q(1/34)
        for i in range(1, 16):
            raw[i] = (_q_normal(i, den) + _q_normal(i + 1, den)) / 2
        neg_scale = -raw[0]
        pos_scale = raw[15]
        out = []
        for i in range(16):
            if i < 8:
                out.append(raw[i] / neg_scale)
            elif i == 8:
                out.append(mpmath.mpf(0))
            else:
                out.append(raw[i] / pos_scale)
    return out


def nf4_codebook() -> np.ndarray:
    """The NF4 table rounded to FP32 (RNE), as float32[16] (reading R(4))."""
    vals = []
    for v in nf4_codebook_exact():
        d = float(v)  # correctly rounded to binary64 by mpmath
        f = np.float32(d)  # RNE binary64 -> binary32
        # Guard against double rounding: the binary64 value must not sit on a binary32 tie.
        assert abs(float(f) - d) != 0.5 * float(np.spacing(np.abs(f))) or d == 0.0
        vals.append(f)
    return np.array(vals, dtype=np.float32)


# --------------------------------------------------------------------------------------
# First level: blockwise absmax + nearest NF4 level
# --------------------------------------------------------------------------------------


def nearest_level(rho: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Index of the NF4 level nearest to each rho ([65B] "Quantization in one paragraph":
    store the index of the level nearest to x/c).  Brute force over all 16 levels; ties go
    to the lower index (reading: the pages do not say).

    Distances are taken in FP64.  Rounding is monotonic, so an FP64 distance can make two
    distinct distances equal but never reverse their order; every FP64 tie is therefore
    settled again with exact rational distances (rho and the levels are binary fractions).
    A false tie happens when a tiny rho sits next to a midpoint at 0 (the INT4 table)."""
    rho = np.asarray(rho, dtype=np.float32).astype(np.float64)
    t = table.astype(np.float64)
    out = np.empty(rho.shape, dtype=np.uint8)
    flat_in = rho.reshape(-1)
    flat_out = out.reshape(-1)
    chunk = 1 << 20
    exact_t = [Fraction(float(v)) for v in t]
    for s in range(0, flat_in.size, chunk):
        r = flat_in[s : s + chunk]
        dist = np.abs(r[:, None] - t[None, :])
        best = np.argmin(dist, axis=1)  # first minimum = lowest index
        tied = np.nonzero(np.sum(dist == dist[np.arange(r.size), best][:, None], axis=1) > 1)[0]
        for i in tied:
            x = Fraction(float(r[i]))
            d = [abs(x - v) for v in exact_t]
            best[i] = d.index(min(d))
        flat_out[s : s + chunk] = best
    return out


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """Pack 4-bit codes, row-major order, two per byte.

    Layout (a format choice; the pages fix none): each aligned run of 8 consecutive
    weights e0..e7 occupies 4 bytes, byte i = e_i | e_{i+4} << 4 (i = 0..3)."""
    c = np.asarray(codes, dtype=np.uint8).reshape(-1)
    assert c.size % 8 == 0
    g = c.reshape(-1, 8).astype(np.uint16)
    packed = (g[:, 0:4] | (g[:, 4:8] << 4)).astype(np.uint8)
    return packed.reshape(-1)


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    """Inverse of :func:`pack_codes`."""
    p = np.asarray(packed, dtype=np.uint8).reshape(-1, 4)
    lo = p & 0x0F
    hi = p >> 4
    return np.concatenate([lo, hi], axis=1).reshape(-1).astype(np.uint8)


# --------------------------------------------------------------------------------------
# OCP FP8 E4M3 (the 8-bit float used for the double-quantized constants)
# --------------------------------------------------------------------------------------


def e4m3_value(code) -> np.ndarray:
    """Value of an OCP E4M3 ("E4M3FN") bit pattern as float64: sign bit, 4 exponent bits
    (bias 7), 3 mantissa bits; exponent 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN."""
    b = np.asarray(code, dtype=np.int64)
    sign = np.where((b >> 7) & 1, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = b & 0x7
    mag = np.where(e == 0, (m / 8.0) * 2.0**-6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7))
    val = sign * mag
    return np.where((e == 15) & (m == 7), np.nan, val)


_E4M3_POS_CODES = np.arange(0x00, 0x7F, dtype=np.int64)  # 0x00..0x7E: all finite non-negative
_E4M3_POS_VALS = e4m3_value(_E4M3_POS_CODES)


def e4m3_encode(s: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest finite E4M3 value, ties to the even code.

    Reading: the 8-bit format of the double-quantized constants is OCP FP8 E4M3 (the
    pages say "8-bit FP8" / "8-bit floats"; [Consumer] says "8-bit integers").  Brute force
    over the 127 finite magnitudes; the sign bit is the sign of s (so tiny negatives give
    0x80).  Values beyond 448 go to 448 (nearest finite)."""
    s = np.asarray(s, dtype=np.float32)
    flat = s.reshape(-1).astype(np.float64)
    neg = np.signbit(s.reshape(-1))
    mag = np.abs(flat)
    out = np.empty(flat.shape, dtype=np.uint8)
    chunk = 1 << 16
    for st in range(0, flat.size, chunk):
        a = mag[st : st + chunk]
        dist = np.abs(a[:, None] - _E4M3_POS_VALS[None, :])
        first = np.argmin(dist, axis=1)
        dmin = dist[np.arange(a.size), first]
        nxt = np.minimum(first + 1, _E4M3_POS_VALS.size - 1)
        tie = (nxt != first) & (dist[np.arange(a.size), nxt] == dmin)
        pick = np.where(tie & (first % 2 == 1), nxt, first)
        out[st : st + chunk] = pick.astype(np.uint8)
    out = np.where(neg, out | 0x80, out).astype(np.uint8)
    return out.reshape(s.shape)


# --------------------------------------------------------------------------------------
# Format variants: other 16-level codebooks and other second-level formats
# --------------------------------------------------------------------------------------

CODEBOOKS = ("nf4", "int4", "fp4")
DQ_FORMATS = ("e4m3", "e5m2", "int8", "none")
E5M2_MAX = 57344.0  # largest finite OCP FP8 E5M2 value (S.11110.11 = 1.75 * 2^15)
INT8_MAX = 127.0


def codebook(name: str = "nf4") -> np.ndarray:
    """16 ascending FP32 levels of a first-level codebook (absmax-normalized to [-1, 1]).

    nf4  : the NormalFloat levels (:func:`nf4_codebook`).
    int4 : standard 4-bit integer quantization, 16 evenly spaced levels over the range
           ([4-Bit] Sec. 2 "1. 4-bit NormalFloat": INT4 divides the range into equal steps;
           reading: the 16 levels -1 + 2 i / 15, so both ends are exact and there is no 0).
    fp4  : the magnitudes of a 4-bit float with 2 exponent and 1 mantissa bit (E2M1:
           0, 0.5, 1, 1.5, 2, 3, 4, 6), both signs, scaled by 1/6 so the ends are +-1; +0 and
           -0 are one level, so the 16th entry repeats +1 (it is never nearest first).
    Each value is its float64 rounded once to FP32."""
    if name == "nf4":
        return nf4_codebook()
    if name == "int4":
        return np.array([np.float32((2.0 * i - 15.0) / 15.0) for i in range(16)], dtype=np.float32)
    if name == "fp4":
        mags = [6.0, 4.0, 3.0, 2.0, 1.5, 1.0, 0.5]
        vals = [-m / 6.0 for m in mags] + [0.0] + [m / 6.0 for m in reversed(mags)] + [1.0]
        return np.array([np.float32(v) for v in vals], dtype=np.float32)
    raise ValueError(name)


def e5m2_value(code) -> np.ndarray:
    """Value of an OCP E5M2 bit pattern as float64: sign, 5 exponent bits (bias 15), 2
    mantissa bits; exponent 0 is subnormal (m/4 * 2^-14); exponent 31 is Inf/NaN."""
    b = np.asarray(code, dtype=np.int64)
    sign = np.where((b >> 7) & 1, -1.0, 1.0)
    e = (b >> 2) & 0x1F
    m = b & 0x3
    mag = np.where(e == 0, (m / 4.0) * 2.0**-14, (1.0 + m / 4.0) * np.exp2(e.astype(np.float64) - 15))
    return np.where(e == 31, np.nan, sign * mag)


_E5M2_POS_CODES = np.arange(0x00, 0x7C, dtype=np.int64)  # 0x00..0x7B: all finite non-negative
_E5M2_POS_VALS = e5m2_value(_E5M2_POS_CODES)


def e5m2_encode(s: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest finite E5M2 value, ties to the even code, beyond
    57344 to 57344; the sign bit is the sign of s.  Brute force over the 124 finite
    magnitudes, as :func:`e4m3_encode`."""
    s = np.asarray(s, dtype=np.float32)
    flat = s.reshape(-1).astype(np.float64)
    neg = np.signbit(s.reshape(-1))
    mag = np.abs(flat)
    out = np.empty(flat.shape, dtype=np.uint8)
    for st in range(0, flat.size, 1 << 16):
        a = mag[st : st + (1 << 16)]
        dist = np.abs(a[:, None] - _E5M2_POS_VALS[None, :])
        first = np.argmin(dist, axis=1)
        dmin = dist[np.arange(a.size), first]
        nxt = np.minimum(first + 1, _E5M2_POS_VALS.size - 1)
        tie = (nxt != first) & (dist[np.arange(a.size), nxt] == dmin)
        out[st : st + (1 << 16)] = np.where(tie & (first % 2 == 1), nxt, first).astype(np.uint8)
    out = np.where(neg, out | 0x80, out).astype(np.uint8)
    return out.reshape(s.shape)


def int8_encode(s: np.ndarray) -> np.ndarray:
    """Symmetric 8-bit integer code of float32 values: round half to even, clamp to
    [-127, 127], stored as the two's-complement byte."""
    q = np.clip(np.rint(np.asarray(s, dtype=np.float32).astype(np.float64)), -INT8_MAX, INT8_MAX)
    return q.astype(np.int64).astype(np.int8).view(np.uint8)


# --------------------------------------------------------------------------------------
# BF16 rounding
# --------------------------------------------------------------------------------------


def bf16_round_bits(x) -> np.ndarray:
    """bfloat16 bit patterns of float32 values, round-to-nearest-even (finite inputs)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------------------
# Quantize: absmax NF4 + double quantization
# --------------------------------------------------------------------------------------


def quantize(W: np.ndarray, blocks: np.ndarray | None = None, codebook_name: str = "nf4",
             dq: str = "e4m3") -> dict:
    """Quantize an FP32 weight matrix W[d_out, d_in] (d_in % 64 == 0).

    `blocks` (optional boolean mask over the flattened 64-blocks) restricts which blocks
    get their 4-bit codes computed (others hold 255); the constants c1, mu, c2s and code8
    always cover the whole tensor, since the mean and the 256-groups span it.

    Steps, in the pages' order:
      1. Blocks of 64 consecutive row-major weights; c1 = max |w| per block
         ([65B] "Quantization in one paragraph").
      2. rho = fl32(w / c1); code = index of the nearest NF4 level (ties to the lower
         index).  An all-zero block (c1 = 0) gets code 8, the exact-zero level (reading).
      3. Double quantization ([4-Bit] Sec. 2 "2. Double Quantization"; [65B] "Double
         quantization"): subtract the mean of the constants first.  Reading: one mean per
         tensor over all its c1, mu = fl32(fl64(exact sum) / n_blocks).
      4. d = fl32(c1 - mu); groups of 256 consecutive constants (flattened block order);
         per group c2s = fl32(max|d| / 448) is the FP32 second-level constant, and
         code8 = E4M3_RNE(fl32(d / c2s)) (code8 = 0 when c2s == 0).
    Returns a dict of the stored buffers plus the transient c1 and the unpacked codes.

    Format variants (the error study of the pages' comparisons: [4-Bit] Sec. 2 "1. 4-bit
    NormalFloat" against INT4 and FP4; Sec. 2 "2. Double Quantization" and [Consumer] FAQ
    for the 8-bit format of the constants, which the pages call both "8-bit floats" and
    "8-bit integers"; [4-Bit] Sec. 2 for FP32 constants without double quantization):
      codebook_name : "nf4" (default), "int4" or "fp4" (:func:`codebook`).  An all-zero
                      block takes the code of the level nearest 0 (ties low): 8 for NF4.
      dq            : "e4m3" (default), "e5m2" (c2s = max|d| / 57344), "int8" (c2s =
                      max|d| / 127, round half to even), or "none": no mean, no second
                      level; code8 then holds the FP32 c1 themselves.
    """
    W = np.asarray(W, dtype=np.float32)
    assert W.ndim == 2 and W.shape[1] % BLOCK1 == 0
    if not np.all(np.isfinite(W)):
        raise ValueError("non-finite weight")
    d_out, d_in = W.shape
    table = codebook(codebook_name)
    sel = None if blocks is None else np.asarray(blocks, dtype=bool).reshape(-1)

    blocks = W.reshape(-1, BLOCK1)
    c1 = np.max(np.abs(blocks), axis=1).astype(np.float32)
    n_blocks = c1.size

    zero_code = int(nearest_level(np.zeros(1, np.float32), table)[0])
    codes = np.full(blocks.shape, zero_code, dtype=np.uint8)
    nz = c1 > 0
    if sel is not None:
        codes[~sel] = 255
        nz = nz & sel
    rho = blocks[nz] / c1[nz][:, None]  # float32 / float32: one IEEE rounding
    codes[nz] = nearest_level(rho, table)

    fmt = {"codebook": codebook_name, "dq": dq}
    if dq == "none":
        return {"d_out": d_out, "d_in": d_in, "codes": codes.reshape(d_out, d_in),
                "packed": pack_codes(codes).reshape(d_out, d_in // 2) if sel is None else None,
                "c1": c1, "mu": np.float32(0.0), "code8": c1.copy(), "c2s": np.zeros(0, np.float32), **fmt}
    top, enc = {"e4m3": (E4M3_MAX, e4m3_encode), "e5m2": (E5M2_MAX, e5m2_encode), "int8": (INT8_MAX, int8_encode)}[dq]

    mu = np.float32(math.fsum(c1.astype(np.float64).tolist()) / n_blocks)

    d = (c1 - mu).astype(np.float32)
    n_groups = -(-n_blocks // BLOCK2)
    c2s = np.zeros(n_groups, dtype=np.float32)
    code8 = np.zeros(n_blocks, dtype=np.uint8)
    for g in range(n_groups):
        seg = d[g * BLOCK2 : (g + 1) * BLOCK2]
        m = np.max(np.abs(seg))
        c2 = np.float32(m / np.float32(top))
        c2s[g] = c2
        if c2 > 0:
            code8[g * BLOCK2 : (g + 1) * BLOCK2] = enc((seg / c2).astype(np.float32))
    return {
        **fmt,
        "d_out": d_out,
        "d_in": d_in,
        "codes": codes.reshape(d_out, d_in),
        "packed": pack_codes(codes).reshape(d_out, d_in // 2) if sel is None else None,
        "c1": c1,
        "mu": mu,
        "code8": code8,
        "c2s": c2s,
    }


def decode_scales(code8: np.ndarray, c2s: np.ndarray, mu, dq: str = "e4m3") -> np.ndarray:
    """Recovered first-level constants: c1_hat = fl32(fl32(v(code8) * c2s) + mu), v the value
    of the 8-bit code (E4M3 by default, E5M2 or the signed integer); for dq = "none" the
    stored FP32 constants themselves.

    Two separate FP32 roundings, undoing the mean shift and the second-level scaling of
    [4-Bit] Sec. 2 "2. Double Quantization" / [65B] "Double quantization"."""
    if dq == "none":
        return np.asarray(code8, dtype=np.float32).copy()
    code8 = np.asarray(code8, dtype=np.uint8)
    n = code8.size
    grp = np.arange(n) // BLOCK2
    if dq == "e4m3":
        v = e4m3_value(code8).astype(np.float32)  # every finite E4M3 value is exact in FP32
    elif dq == "e5m2":
        v = e5m2_value(code8).astype(np.float32)
    else:
        v = code8.view(np.int8).astype(np.float32)
    prod = (v * np.asarray(c2s, dtype=np.float32)[grp]).astype(np.float32)
    return (prod + np.float32(mu)).astype(np.float32)


def dequantize_bf16_bits(q: dict) -> np.ndarray:
    """Dequantized weights as BF16 bit patterns [d_out, d_in]:
    w_hat = bf16(fl32(q[code] * c1_hat)) -- a lookup and a multiply ([65B] "Quantization
    in one paragraph"), rounded to the BF16 compute type ([4-Bit] Sec. 3).
    Blocks whose codes were not computed (code 255) decode to NaN."""
    table = np.concatenate([codebook(q.get("codebook", "nf4")), np.full(240, np.nan, np.float32)])
    c1h = decode_scales(q["code8"], q["c2s"], q["mu"], q.get("dq", "e4m3"))
    codes = q["codes"].reshape(-1, BLOCK1)
    vals = (table[codes] * c1h[:, None]).astype(np.float32)
    bits = bf16_round_bits(np.where(np.isnan(vals), 0, vals))
    bits = np.where(np.isnan(vals), np.uint16(0x7FC0), bits)
    return bits.reshape(q["d_out"], q["d_in"])


def dequantize_f64(q: dict) -> np.ndarray:
    return bf16_bits_to_f32(dequantize_bf16_bits(q)).astype(np.float64)


# --------------------------------------------------------------------------------------
# LoRA-augmented linear: forward and backward (FP64 over the exact BF16 inputs)
# --------------------------------------------------------------------------------------


def lora_fwd(W_hat: np.ndarray, X: np.ndarray, A: np.ndarray, B: np.ndarray, alpha: float, r: int):
    """Forward of the frozen quantized linear with its adapter.

    [65B] "Prerequisite: LoRA" and "Where the gradients actually go": h = deq(W) x + B A x;
    [4-Bit] Sec. 3 scales the adapter branch by alpha/r.  Row-major batch form:
      T = X A^T  [M, r],   Y = X W_hat^T + (alpha/r) T B^T  [M, d_out].
    W_hat [d_out, d_in], X [M, d_in], A [r, d_in], B [d_out, r]; all float64.
    Returns (Y, T)."""
    s = float(alpha) / float(r)
    T = X @ A.T
    Y = X @ W_hat.T + s * (T @ B.T)
    return Y, T


def lora_bwd(W_hat: np.ndarray, X: np.ndarray, dY: np.ndarray, A: np.ndarray, B: np.ndarray, alpha: float, r: int):
    """Backward ([65B] "Where the gradients actually go"): the input gradient runs through
    the dequantized frozen weights, and only the adapters receive parameter gradients.
      G  = dY B                    [M, r]
      dX = dY W_hat + (alpha/r) G A   [M, d_in]   (chain rule through both branches)
      dA = (alpha/r) G^T X         [r, d_in]
      dB = (alpha/r) dY^T T, T = X A^T   [d_out, r]
    No gradient for W is formed."""
    s = float(alpha) / float(r)
    T = X @ A.T
    G = dY @ B
    dX = dY @ W_hat + s * (G @ A)
    dA = s * (G.T @ X)
    dB = s * (dY.T @ T)
    return dX, dA, dB


# --------------------------------------------------------------------------------------
# Storage sizes
# --------------------------------------------------------------------------------------


def quant_sizes(d_out: int, d_in: int, dq: str = "e4m3") -> dict:
    """Bytes of each stored buffer: 4-bit codes, one 8-bit constant per 64 weights, one
    FP32 second-level constant per 256 constants, and one FP32 mean per tensor; without
    double quantization one FP32 constant per 64 weights and nothing else."""
    n = d_out * d_in
    n_blocks = n // BLOCK1
    n_groups = -(-n_blocks // BLOCK2)
    if dq == "none":
        return {"codes": n // 2, "code8": 4 * n_blocks, "c2s": 0, "mu": 0}
    return {"codes": n // 2, "code8": n_blocks, "c2s": 4 * n_groups, "mu": 4}


def bits_per_param(d_out: int, d_in: int, double_quant: bool = True) -> float:
    """Storage bits per weight.  Without double quantization the constants are FP32 per
    64 weights ([65B] "Double quantization": 4 + 32/64 = 4.5)."""
    n = d_out * d_in
    sz = quant_sizes(d_out, d_in)
    if not double_quant:
        return 8.0 * (sz["codes"] + 4 * (n // BLOCK1)) / n
    return 8.0 * sum(sz.values()) / n


# --------------------------------------------------------------------------------------
# Merge / export: fold the adapter into the dequantized base, optionally re-quantize
# --------------------------------------------------------------------------------------


def bf16_round_f64_bits(x) -> np.ndarray:
    """bfloat16 bit patterns of float64 values, one round-to-nearest-even (finite inputs).

    Rounding float64 -> float32 -> bfloat16 by RNE twice can differ from one rounding.  The
    first step is therefore done by rounding to odd (truncate, then set the last bit when
    the truncation was inexact); a float32 carries 24 >= 2 * 8 + 2 significant bits, so
    the following RNE to bfloat16 equals the direct RNE of x (Boldo and Melquiond,
    "Emulation of FMA and correctly rounded sums: proved algorithms using rounding to odd",
    IEEE Trans. Computers, 2008)."""
    x = np.asarray(x, dtype=np.float64)
    f = x.astype(np.float32)  # RNE
    away = np.abs(f.astype(np.float64)) > np.abs(x)
    f = np.where(away, np.nextafter(f, np.float32(0)), f).astype(np.float32)  # truncation
    inexact = (f.astype(np.float64) != x).astype(np.uint32)
    f = (f.view(np.uint32) | inexact).view(np.float32)
    return bf16_round_bits(f)


def merge(q: dict, A: np.ndarray, B: np.ndarray, alpha: float, r: int):
    """Merged 16-bit weight W' = bf16(w_hat + (alpha/r) B A), d_out x d_in.

    [4-Bit] "Interview questions" (deployment): the base is dequantized back to 16 bits
    and the trained adapter is added, W = W_dequant + (alpha/r) B A, giving an ordinary
    16-bit checkpoint.  [65B] "Pitfalls" and "How it's used in practice": the merge happens
    in 16 bits, never inside the 4-bit format; the merged result may then be quantized
    again (:func:`quantize_bf16`).  The sum is exact in float64 over the BF16 w_hat and the
    BF16 adapters, rounded once to BF16.
    Returns (BF16 bit patterns [d_out, d_in], the float64 values before rounding)."""
    s = float(alpha) / float(r)
    exact = dequantize_f64(q) + s * (np.asarray(B, np.float64) @ np.asarray(A, np.float64))
    return bf16_round_f64_bits(exact), exact


def quantize_bf16(W_bits: np.ndarray, blocks: np.ndarray | None = None, codebook_name: str = "nf4",
                  dq: str = "e4m3") -> dict:
    """Quantize a BF16 weight matrix (bit patterns).  Every BF16 value is exact in FP32,
    so this is :func:`quantize` of the widened values: the 16-bit checkpoint a model ships
    in is quantized as it stands ([4-Bit] Sec. 1: the frozen base lives in 16 bits)."""
    return quantize(bf16_bits_to_f32(W_bits), blocks, codebook_name, dq)


# --------------------------------------------------------------------------------------
# Adapter optimizer step: AdamW with FP32 master weights and moments
# --------------------------------------------------------------------------------------


def adamw_step(master: np.ndarray, m: np.ndarray, v: np.ndarray, grad_bits: np.ndarray, step: int,
               lr: float, beta1: float, beta2: float, eps: float, weight_decay: float):
    """One AdamW step over flat adapter parameters.

    State layout from the pages: every trainable parameter keeps an FP32 master copy, an
    FP32 first moment and an FP32 second moment (12 bytes), next to the 16-bit weight and
    16-bit gradient ("QLoRA: Quantize Base Weights to 4-Bit", Section 1 and Section 4's
    optimizer term; "QLoRA -- Fine-Tuning a 65B Model on One GPU", "Paged optimizers").
    The pages name AdamW but do not print it; the update is the published one
    (Loshchilov and Hutter, "Decoupled Weight Decay Regularization", ICLR 2019, with the
    bias correction of Kingma and Ba, "Adam", ICLR 2015), with the decay scaled by lr:
      theta <- theta (1 - lr wd)
      m <- b1 m + (1 - b1) g,   v <- b2 v + (1 - b2) g^2
      theta <- theta - lr (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps)
    g is the BF16 gradient widened exactly.  Arithmetic in FP64 from the FP32 inputs; the
    three states are returned rounded to FP32 (their storage type) and the working weight
    as BF16 bits of the new FP32 master.
    Returns (master, m, v as float32; param BF16 bits; the FP64 master before rounding)."""
    t = int(step)
    assert t >= 1
    th = np.asarray(master, np.float32).astype(np.float64)
    m0 = np.asarray(m, np.float32).astype(np.float64)
    v0 = np.asarray(v, np.float32).astype(np.float64)
    g = bf16_bits_to_f32(grad_bits).astype(np.float64)
    th = th * (1.0 - lr * weight_decay)
    m1 = beta1 * m0 + (1.0 - beta1) * g
    v1 = beta2 * v0 + (1.0 - beta2) * g * g
    mhat = m1 / (1.0 - beta1**t)
    vhat = v1 / (1.0 - beta2**t)
    th = th - lr * mhat / (np.sqrt(vhat) + eps)
    th32 = th.astype(np.float32)
    return th32, m1.astype(np.float32), v1.astype(np.float32), bf16_round_bits(th32), th


# --------------------------------------------------------------------------------------
# MLP block of a decoder layer: gate, up and down projections, all quantized and adapted
# --------------------------------------------------------------------------------------


def silu(g: np.ndarray) -> np.ndarray:
    """silu(g) = g * sigmoid(g) = g / (1 + e^-g), float64.

    Reading: [65B] "Seeing it in code" puts adapters on gate_proj, up_proj and down_proj, but
    no page states the activation between them; the gated one those names denote is taken,
    H = silu(gate(X)) * up(X), Y = down(H)."""
    g = np.asarray(g, dtype=np.float64)
    return g / (1.0 + np.exp(-g))


def mlp_fwd(Wg_hat, Wu_hat, Wd_hat, X, As, Bs, alpha: float, r: int):
    """Forward of the MLP block, each projection a frozen quantized linear with its adapter
    (:func:`lora_fwd`): G = gate(X), U = up(X), H = silu(G) * U, Y = down(H).
    Wg_hat, Wu_hat [f, d]; Wd_hat [d, f]; X [M, d]; As, Bs in the order gate, up, down.
    Every step exact in float64.  Returns (Y, G, U, H)."""
    G, _ = lora_fwd(Wg_hat, X, As[0], Bs[0], alpha, r)
    U, _ = lora_fwd(Wu_hat, X, As[1], Bs[1], alpha, r)
    H = silu(G) * U
    Y, _ = lora_fwd(Wd_hat, H, As[2], Bs[2], alpha, r)
    return Y, G, U, H


def mlp_bwd(Wg_hat, Wu_hat, Wd_hat, X, dY, As, Bs, alpha: float, r: int):
    """Backward of :func:`mlp_fwd` by the chain rule, the inner activations recomputed from X
    (the gradient checkpointing of [65B] "Seeing it in code"):
      dH = input gradient of down;  with s = sigmoid(G),
      dG = dH * U * s * (1 + G (1 - s)),   dU = dH * G * s;
      dX = (input gradient of gate for dG) + (input gradient of up for dU);
    each projection's adapter gradients as :func:`lora_bwd` gives them.
    Returns (dX, [dA_gate, dA_up, dA_down], [dB_gate, dB_up, dB_down])."""
    _, G, U, H = mlp_fwd(Wg_hat, Wu_hat, Wd_hat, X, As, Bs, alpha, r)
    dH, dA_d, dB_d = lora_bwd(Wd_hat, H, dY, As[2], Bs[2], alpha, r)
    s = 1.0 / (1.0 + np.exp(-G))
    dG = dH * U * s * (1.0 + G * (1.0 - s))
    dU = dH * G * s
    dX_g, dA_g, dB_g = lora_bwd(Wg_hat, X, dG, As[0], Bs[0], alpha, r)
    dX_u, dA_u, dB_u = lora_bwd(Wu_hat, X, dU, As[1], Bs[1], alpha, r)
    return dX_g + dX_u, [dA_g, dA_u, dA_d], [dB_g, dB_u, dB_d]
