"""GPU parity of the export path: the merged 16-bit weight bf16(w_hat + (alpha/r) B A) and
the quantization of BF16 weights, through the C ABI, against the CPU oracle.

Merge tolerance, derived from the arithmetic.  The library forms v = fl32(w_hat + s * acc)
with acc the FP32 MFMA sum of r exact BF16 products and s = fl32(alpha / r), then rounds v
to BF16 once.  With u = 2^-24:
    |v - exact| <= s (r + 1) u sum_j |B[n][j] A[j][k]| + u |v|,
so v and the exact value round to the same BF16 pattern unless a BF16 rounding boundary
lies within that distance of the exact value.  The test therefore demands equality
everywhere except where the oracle's exact value is within
    bound = 4 u (s (r + 1) (|B| |A|) + |exact|)      (a 4x margin)
of the midpoint between the two patterns, and there the two must be adjacent patterns.
BF16 quantization is bit-exact: both sides quantize the same exact FP32 values."""

import numpy as np
import pytest
import torch

import oracle as O
from bit_nf4_quantized_dq_amd import inputs as I

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def _f64_bits(b):
    return O.bf16_bits_to_f32(b).astype(np.float64)


def _assert_merge_parity(got, ref, exact, A64, B64, s, r):
    diff = got != ref
    n_diff = int(diff.sum())
    if n_diff == 0:
        return
    bound = 2.0**-22 * (s * (r + 1) * (np.abs(B64) @ np.abs(A64)) + np.abs(exact))
    fg, fr = _f64_bits(got[diff]), _f64_bits(ref[diff])
    ex, bd = exact[diff], bound[diff]
    # adjacent patterns: no BF16 value strictly between them
    ulp = np.maximum(np.spacing(np.abs(fr).astype(np.float32)).astype(np.float64) * 2.0**16, 2.0**-133)
    assert np.all(np.abs(fg - fr) <= ulp), "merged value off by more than one BF16 step"
    mid = 0.5 * (fg + fr)
    assert np.all(np.abs(mid - ex) <= bd), "mismatch away from a rounding boundary"
    assert n_diff <= max(4, diff.size // 1000), f"{n_diff} rounding-boundary mismatches"


MERGE_CASES = [
    # cfg, d_out, d_in, r, alpha, B std (the trained adapter's scale)
    (1, 256, 256, 8, 16.0, 0.01),
    (2, 4096, 4096, 16, 32.0, 0.01),
    (9, 272, 320, 40, 80.0, 0.05),   # ragged row and column tiles, 3 rank chunks
    (9, 144, 192, 5, 7.0, 0.05),     # r % 8 != 0: element loads of B, padded rank chunk
    (9, 16, 64, 128, 256.0, 0.05),   # the largest rank on the smallest tensor
    (9, 400, 1088, 17, 3.0, 0.2),    # r = 17: two chunks, the second nearly empty
]


@pytest.mark.parametrize("cfg,d_out,d_in,r,alpha,bstd", MERGE_CASES)
def test_merge_parity(gpu_lib, cfg, d_out, d_in, r, alpha, bstd):
    from bit_nf4_quantized_dq_amd import merge, quantize

    print(f"merge cfg={cfg} {d_out}x{d_in} r={r}", flush=True)
    W = I.weight(cfg, 0, d_out, d_in, 0.02)
    A = I.lora_A(cfg, 0, r, d_in)
    B = (I.lora_B(cfg, 0, d_out, r).float() * (bstd / 0.01)).to(torch.bfloat16)
    oq = O.quantize(W.numpy())
    A64, B64 = A.double().numpy(), B.double().numpy()
    ref, exact = O.merge(oq, A64, B64, alpha, r)
    q = quantize(W.cuda())
    out = merge(q, A.cuda(), B.cuda(), alpha)
    torch.cuda.synchronize()
    got = _bits(out)
    _assert_merge_parity(got, ref, exact, A64, B64, alpha / r, r)
    # the adapter really moved the weights (a dropped B A would leave the base)
    assert np.mean(got != O.dequantize_bf16_bits(oq)) > 0.2


def test_merge_adapter_in_isolation(gpu_lib):
    """W = 0: the merge is bf16(s B A) alone, so a wrong scale, a transposed operand or a
    wrong rank chunk shows at full size."""
    from bit_nf4_quantized_dq_amd import merge, quantize

    d_out, d_in, r, alpha = 272, 576, 24, 12.0
    W = torch.zeros(d_out, d_in)
    A = I.lora_A(9, 1, r, d_in)
    B = I.lora_B(9, 1, d_out, r)
    oq = O.quantize(W.numpy())
    A64, B64 = A.double().numpy(), B.double().numpy()
    ref, exact = O.merge(oq, A64, B64, alpha, r)
    out = merge(quantize(W.cuda()), A.cuda(), B.cuda(), alpha)
    torch.cuda.synchronize()
    _assert_merge_parity(_bits(out), ref, exact, A64, B64, alpha / r, r)
    assert np.count_nonzero(ref) > 0.99 * ref.size


def test_merge_zero_adapter_is_dequantize(gpu_lib):
    from bit_nf4_quantized_dq_amd import dequantize, merge, quantize

    W = I.weight(9, 2, 528, 448, 0.02)
    q = quantize(W.cuda())
    out = merge(q, torch.zeros(16, 448, dtype=torch.bfloat16, device="cuda"),
                torch.zeros(528, 16, dtype=torch.bfloat16, device="cuda"), 32.0)
    w = dequantize(q)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(out), _bits(w))
    assert np.array_equal(_bits(out), O.dequantize_bf16_bits(O.quantize(W.numpy())))


BQ_SHAPES = [(1, 256, 256), (2, 4096, 4096), (9, 272, 320), (9, 16, 64)]


@pytest.mark.parametrize("cfg,d_out,d_in", BQ_SHAPES)
def test_quantize_bf16_bit_exact(gpu_lib, cfg, d_out, d_in):
    from bit_nf4_quantized_dq_amd import quantize_bf16

    Wb = I.weight(cfg, 3, d_out, d_in, 0.02).to(torch.bfloat16)
    oq = O.quantize_bf16(_bits(Wb))
    q = quantize_bf16(Wb.cuda())
    torch.cuda.synchronize()
    assert np.array_equal(q.codes.cpu().numpy(), oq["packed"].reshape(-1))
    assert np.array_equal(q.code8.cpu().numpy(), oq["code8"])
    assert np.array_equal(q.c2s.cpu().numpy().view(np.uint32), oq["c2s"].view(np.uint32))
    assert q.mu.cpu().numpy().view(np.uint32)[0] == np.float32(oq["mu"]).view(np.uint32)


def test_merge_then_requantize_chain(gpu_lib):
    """quantize -> merge -> quantize_bf16 on both sides.  The adapters are small dyadic
    numbers (A = a 2^-6, B = b 2^-8, |a|, |b| <= 8), so every sum is exact in FP32 and the
    merged weights agree bit for bit before they are quantized again."""
    from bit_nf4_quantized_dq_amd import merge, quantize, quantize_bf16

    d_out, d_in, r, alpha = 512, 1024, 16, 32.0
    W = I.weight(9, 4, d_out, d_in, 0.02)
    g = torch.Generator().manual_seed(9044)
    A = (torch.randint(-8, 9, (r, d_in), generator=g).float() * 2.0**-6).to(torch.bfloat16)
    B = (torch.randint(-8, 9, (d_out, r), generator=g).float() * 2.0**-8).to(torch.bfloat16)
    oq = O.quantize(W.numpy())
    ref, _ = O.merge(oq, A.double().numpy(), B.double().numpy(), alpha, r)
    merged = merge(quantize(W.cuda()), A.cuda(), B.cuda(), alpha)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(merged), ref)
    oq2 = O.quantize_bf16(ref)
    q2 = quantize_bf16(merged)
    torch.cuda.synchronize()
    assert np.array_equal(q2.codes.cpu().numpy(), oq2["packed"].reshape(-1))
    assert np.array_equal(q2.code8.cpu().numpy(), oq2["code8"])
    assert np.array_equal(q2.c2s.cpu().numpy().view(np.uint32), oq2["c2s"].view(np.uint32))
    assert q2.mu.cpu().numpy().view(np.uint32)[0] == np.float32(oq2["mu"]).view(np.uint32)
