"""CPU-side checks of the C-ABI library: it loads, exports every symbol the header declares,
and its host-only entry points (sizes, codebook, argument validation) behave.  No GPU
compute is called: every error path tested here returns before any launch."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O
from bit_nf4_quantized_dq_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qlora.h")


@pytest.fixture(scope="module")
def L():
    return B.load_library()


def test_every_declared_symbol_is_exported(L):
    text = open(HEADER).read()
    names = sorted(set(re.findall(r"\b(qlora_[a-z0-9_]+)\s*\(", text)))
    assert len(names) == 24
    for n in names:
        assert hasattr(L, n), n


def test_codebook_equals_oracle_bit_for_bit():
    lib_q = np.array(B.nf4_codebook(), dtype=np.float32)
    assert np.array_equal(lib_q.view(np.uint32), O.nf4_codebook().view(np.uint32))


@pytest.mark.parametrize("shape", [(256, 256), (4096, 4096), (1024, 4096), (14336, 4096), (4096, 14336), (272, 320)])
def test_quant_sizes_match_oracle(shape):
    a, b, c = B.quant_sizes(*shape)
    sz = O.quant_sizes(*shape)
    assert (a, b, c) == (sz["codes"], sz["code8"], sz["c2s"])


def test_bits_per_param_from_library_sizes():
    a, b, c = B.quant_sizes(4096, 4096)
    bpp = 8.0 * (a + b + c + 4) / (4096 * 4096)
    assert round(bpp, 3) == 4.127


def _wq(d_out=256, d_in=256, b1=64, b2=256, cb=0, dq=0, c2s=4096):
    dummy = ctypes.c_void_p(4096)  # never dereferenced: validation fails first
    return B._Nf4dq(dummy, dummy, ctypes.c_void_p(c2s) if c2s else None, dummy, d_out, d_in, b1, b2, cb, dq)


def test_shape_and_argument_errors_before_launch(L):
    dummy = ctypes.c_void_p(4096)
    ws = ctypes.c_void_p(8192)
    assert L.qlora_linear_fwd(ctypes.byref(_wq(d_in=100)), dummy, 4, dummy, dummy, 8, 16.0, dummy, None, ws, 1 << 20, None) == -2
    assert L.qlora_linear_fwd(ctypes.byref(_wq(d_out=250)), dummy, 4, dummy, dummy, 8, 16.0, dummy, None, ws, 1 << 20, None) == -2
    assert L.qlora_linear_fwd(ctypes.byref(_wq(b1=32)), dummy, 4, dummy, dummy, 8, 16.0, dummy, None, ws, 1 << 20, None) == -3
    assert L.qlora_linear_fwd(ctypes.byref(_wq()), dummy, 0, dummy, dummy, 8, 16.0, dummy, None, ws, 1 << 20, None) == -1
    # M below 2^24: [M, r] operands stay within the 4 GiB reach of a buffer descriptor
    assert L.qlora_linear_fwd(ctypes.byref(_wq()), dummy, 1 << 24, dummy, dummy, 8, 16.0, dummy, None, ws, 1 << 40, None) == -1
    assert L.qlora_linear_bwd(ctypes.byref(_wq()), dummy, dummy, 1 << 24, dummy, dummy, 8, 16.0, None, dummy, dummy, dummy,
                              ws, 1 << 40, None) == -1
    # the workspace: misaligned is an argument error, too small a workspace error
    assert L.qlora_linear_fwd(ctypes.byref(_wq()), dummy, 4, dummy, dummy, 8, 16.0, dummy, None, ctypes.c_void_p(8200),
                              1 << 20, None) == -1
    assert L.qlora_linear_fwd(ctypes.byref(_wq()), dummy, 4, dummy, dummy, 0, 16.0, dummy, None, ws, 1 << 20, None) == -1
    assert L.qlora_linear_fwd(ctypes.byref(_wq()), dummy, 4, dummy, dummy, 129, 16.0, dummy, None, ws, 1 << 20, None) == -1
    assert L.qlora_linear_fwd(ctypes.byref(_wq()), dummy, 4, dummy, dummy, 8, float("nan"), dummy, None, ws, 1 << 20, None) == -1
    assert L.qlora_linear_fwd(ctypes.byref(_wq()), None, 4, dummy, dummy, 8, 16.0, dummy, None, ws, 1 << 20, None) == -1
    assert L.qlora_linear_fwd(ctypes.byref(_wq()), dummy, 4, dummy, dummy, 8, 16.0, dummy, None, ws, 16, None) == -5
    assert L.qlora_linear_fwd(ctypes.byref(_wq()), dummy, 4, dummy, dummy, 8, 16.0, dummy, None, None, 1 << 20, None) == -5
    assert L.qlora_linear_bwd(ctypes.byref(_wq()), dummy, dummy, 4, dummy, dummy, 8, 16.0, None, dummy, dummy, None, ws, 1 << 20, None) == -1
    assert L.qlora_linear_bwd(ctypes.byref(_wq()), dummy, dummy, 4, dummy, dummy, 8, 16.0, None, dummy, dummy, dummy, ws, 8, None) == -5
    assert L.qlora_quantize(dummy, ctypes.byref(_wq()), None, ws, 8, None) == -5
    assert L.qlora_quantize(None, ctypes.byref(_wq()), None, ws, 1 << 20, None) == -1
    assert L.qlora_quantize(ctypes.c_void_p(4100), ctypes.byref(_wq()), None, ws, 1 << 20, None) == -1  # misaligned
    assert L.qlora_dequantize(None, dummy, None) == -1
    assert L.qlora_quantize_bf16(dummy, ctypes.byref(_wq()), None, ws, 8, None) == -5
    assert L.qlora_quantize_bf16(ctypes.c_void_p(4098), ctypes.byref(_wq()), None, ws, 1 << 20, None) == -1
    assert L.qlora_quantize_bf16(dummy, ctypes.byref(_wq(d_in=96)), None, ws, 1 << 20, None) == -2
    assert L.qlora_merge(ctypes.byref(_wq()), dummy, dummy, 0, 16.0, dummy, None) == -1
    assert L.qlora_merge(ctypes.byref(_wq()), dummy, dummy, 129, 16.0, dummy, None) == -1
    assert L.qlora_merge(ctypes.byref(_wq()), dummy, dummy, 8, float("inf"), dummy, None) == -1
    assert L.qlora_merge(ctypes.byref(_wq()), dummy, None, 8, 16.0, dummy, None) == -1
    assert L.qlora_merge(ctypes.byref(_wq()), dummy, ctypes.c_void_p(4098), 8, 16.0, dummy, None) == -1  # B misaligned
    assert L.qlora_merge(ctypes.byref(_wq()), dummy, dummy, 8, 16.0, ctypes.c_void_p(4098), None) == -1
    assert L.qlora_merge(ctypes.byref(_wq(d_out=250)), dummy, dummy, 8, 16.0, dummy, None) == -2
    assert L.qlora_merge(ctypes.byref(_wq(b1=32)), dummy, dummy, 8, 16.0, dummy, None) == -3
    # formats: unknown codebook or second-level format, missing c2s where it is needed
    assert L.qlora_dequantize(ctypes.byref(_wq(cb=3)), dummy, None) == -3
    assert L.qlora_dequantize(ctypes.byref(_wq(dq=4)), dummy, None) == -3
    assert L.qlora_dequantize(ctypes.byref(_wq(dq=-1)), dummy, None) == -3
    assert L.qlora_dequantize(ctypes.byref(_wq(dq=1, c2s=0)), dummy, None) == -1
    assert L.qlora_merge(ctypes.byref(_wq(cb=7)), dummy, dummy, 8, 16.0, dummy, None) == -3
    assert L.qlora_linear_fwd(ctypes.byref(_wq(dq=9)), dummy, 4, dummy, dummy, 8, 16.0, dummy, None, ws, 1 << 20, None) == -3
    n = ctypes.c_size_t()
    assert L.qlora_workspace_size_fmt(1, 4, 256, 256, 8, 7, ctypes.byref(n)) == -3
    f16 = (ctypes.c_float * 16)()
    assert L.qlora_codebook(3, f16) == -1 and L.qlora_codebook(0, None) == -1
    f = ctypes.c_float
    ok = dict(lr=f(1e-3), b1=f(0.9), b2=f(0.999), eps=f(1e-8), wd=f(0.0))
    def adamw(master=dummy, g=dummy, p=dummy, n=16, step=1, **kw):
        a = dict(ok, **{k: f(x) for k, x in kw.items()})
        return L.qlora_adamw_step(master, dummy, dummy, g, p, n, step, a["lr"], a["b1"], a["b2"], a["eps"], a["wd"], None)
    assert adamw(n=0) == 0 and adamw(master=None, n=0) == 0  # no-op
    assert adamw(n=-1) == -1 and adamw(step=0) == -1
    assert adamw(master=None) == -1 and adamw(g=None) == -1
    assert adamw(master=ctypes.c_void_p(4100)) == -1 and adamw(g=ctypes.c_void_p(4098)) == -1
    assert adamw(p=ctypes.c_void_p(4098)) == -1
    assert adamw(lr=-1.0) == -1 and adamw(lr=float("nan")) == -1 and adamw(b1=1.0) == -1 and adamw(b2=-0.1) == -1
    assert adamw(eps=0.0) == -1 and adamw(wd=-0.5) == -1 and adamw(wd=float("inf")) == -1


def test_workspace_head_and_init_errors(L):
    """Every workspace starts with the counter head: sizes include it, the init call checks
    its arguments before any launch."""
    head = 524288
    n = ctypes.c_size_t()
    for op in (0, 1, 2):
        assert L.qlora_workspace_size(op, 4, 256, 256, 8, ctypes.byref(n)) == 0 and n.value > head
    assert L.qlora_workspace_init(None, 1 << 20, None) == -1
    assert L.qlora_workspace_init(ctypes.c_void_p(8200), 1 << 20, None) == -1
    assert L.qlora_workspace_init(ctypes.c_void_p(8192), head - 1, None) == -5


def test_noalloc_forward_errors_before_launch(L):
    """The forward on the fixed scratch validates as qlora_linear_fwd does, and refuses a call
    that needs more than its scratch (here the decoded 4096 x 4096 copy at M = 4096) with its
    own status, before any launch or device lookup."""
    dummy = ctypes.c_void_p(4096)
    assert L.qlora_linear_fwd_noalloc(ctypes.byref(_wq(d_in=100)), dummy, 4, dummy, dummy, 8, 16.0, dummy, None, None) == -2
    assert L.qlora_linear_fwd_noalloc(ctypes.byref(_wq()), dummy, 0, dummy, dummy, 8, 16.0, dummy, None, None) == -1
    assert L.qlora_linear_fwd_noalloc(ctypes.byref(_wq()), None, 4, dummy, dummy, 8, 16.0, dummy, None, None) == -1
    assert L.qlora_linear_fwd_noalloc(None, dummy, 4, dummy, dummy, 8, 16.0, dummy, None, None) == -1
    big = _wq(d_out=4096, d_in=4096)
    assert L.qlora_linear_fwd_noalloc(ctypes.byref(big), dummy, 4096, dummy, dummy, 16, 32.0, dummy, None, None) == -7


def test_grouped_forward_errors_before_launch(L):
    """qlora_linear_fwd_multi / qlora_workspace_size_multi reject bad groups on the host."""
    dummy = ctypes.c_void_p(4096)
    ws = ctypes.c_void_p(8192)
    P = ctypes.POINTER(B._Nf4dq)

    def group(*wqs):
        keep = list(wqs)
        return (P * len(keep))(*[ctypes.pointer(w) for w in keep]), keep

    VP = ctypes.c_void_p * 5
    ptrs = VP(dummy, dummy, dummy, dummy, dummy)
    n = ctypes.c_size_t()
    ok, _k1 = group(_wq(), _wq(d_out=512))
    assert L.qlora_workspace_size_multi(2, ok, 4, 8, ctypes.byref(n)) == 0 and n.value >= 256
    assert L.qlora_workspace_size_multi(2, ok, 4, 8, None) == -1
    assert L.qlora_workspace_size_multi(0, ok, 4, 8, ctypes.byref(n)) == -1
    five, _k2 = group(*[_wq() for _ in range(5)])
    assert L.qlora_workspace_size_multi(5, five, 4, 8, ctypes.byref(n)) == -1
    assert L.qlora_linear_fwd_multi(5, five, dummy, 4, ptrs, ptrs, 8, 16.0, ptrs, None, ws, 1 << 20, None) == -1
    mixed, _k3 = group(_wq(), _wq(d_in=512))
    assert L.qlora_workspace_size_multi(2, mixed, 4, 8, ctypes.byref(n)) == -2
    assert L.qlora_linear_fwd_multi(2, mixed, dummy, 4, ptrs, ptrs, 8, 16.0, ptrs, None, ws, 1 << 20, None) == -2
    bad, _k4 = group(_wq(), _wq(b1=32))
    assert L.qlora_linear_fwd_multi(2, bad, dummy, 4, ptrs, ptrs, 8, 16.0, ptrs, None, ws, 1 << 20, None) == -3
    assert L.qlora_linear_fwd_multi(2, ok, None, 4, ptrs, ptrs, 8, 16.0, ptrs, None, ws, 1 << 20, None) == -1
    assert L.qlora_linear_fwd_multi(2, ok, dummy, 4, None, ptrs, 8, 16.0, ptrs, None, ws, 1 << 20, None) == -1
    holes = VP(dummy, None, dummy, dummy, dummy)
    assert L.qlora_linear_fwd_multi(2, ok, dummy, 4, ptrs, ptrs, 8, 16.0, holes, None, ws, 1 << 20, None) == -1
    assert L.qlora_linear_fwd_multi(2, ok, dummy, 4, ptrs, ptrs, 0, 16.0, ptrs, None, ws, 1 << 20, None) == -1
    assert L.qlora_linear_fwd_multi(2, ok, dummy, 4, ptrs, ptrs, 8, 16.0, ptrs, None, ws, 16, None) == -5


def test_mlp_block_errors_before_launch(L):
    """qlora_mlp_* reject shapes that do not chain and missing buffers on the host."""
    dummy = ctypes.c_void_p(4096)
    ws = ctypes.c_void_p(8192)
    VP = ctypes.c_void_p * 3
    ptrs = VP(dummy, dummy, dummy)
    g, u, d = _wq(d_out=512, d_in=256), _wq(d_out=512, d_in=256), _wq(d_out=256, d_in=512)
    n = ctypes.c_size_t()
    assert L.qlora_mlp_workspace_size(1, 64, ctypes.byref(g), ctypes.byref(u), ctypes.byref(d), 8, ctypes.byref(n)) == 0
    fwd_need = n.value
    assert L.qlora_mlp_workspace_size(2, 64, ctypes.byref(g), ctypes.byref(u), ctypes.byref(d), 8, ctypes.byref(n)) == 0
    assert n.value > fwd_need >= 3 * 2 * 64 * 512
    assert L.qlora_mlp_workspace_size(3, 64, ctypes.byref(g), ctypes.byref(u), ctypes.byref(d), 8, ctypes.byref(n)) == -1
    bad_d = _wq(d_out=256, d_in=256)  # down must take d_in = f = 512
    assert L.qlora_mlp_workspace_size(1, 64, ctypes.byref(g), ctypes.byref(u), ctypes.byref(bad_d), 8, ctypes.byref(n)) == -2
    assert L.qlora_mlp_fwd(ctypes.byref(g), ctypes.byref(u), ctypes.byref(bad_d), dummy, 64, ptrs, ptrs, 8, 16.0, dummy,
                           None, None, ws, 1 << 30, None) == -2
    assert L.qlora_mlp_fwd(ctypes.byref(g), ctypes.byref(u), ctypes.byref(d), None, 64, ptrs, ptrs, 8, 16.0, dummy,
                           None, None, ws, 1 << 30, None) == -1
    assert L.qlora_mlp_fwd(ctypes.byref(g), ctypes.byref(u), ctypes.byref(d), dummy, 64, ptrs, ptrs, 8, 16.0, dummy,
                           None, None, ws, 16, None) == -5
    # every adapter pointer is checked before the first launch: a missing or misaligned A[2]
    # (the down projection's, used last) and a missing dA[1] fail up front
    late = VP(dummy, dummy, None)
    assert L.qlora_mlp_fwd(ctypes.byref(g), ctypes.byref(u), ctypes.byref(d), dummy, 64, late, ptrs, 8, 16.0, dummy,
                           None, None, ws, 1 << 30, None) == -1
    odd = VP(dummy, dummy, ctypes.c_void_p(4098))
    assert L.qlora_mlp_fwd(ctypes.byref(g), ctypes.byref(u), ctypes.byref(d), dummy, 64, odd, ptrs, 8, 16.0, dummy,
                           None, None, ws, 1 << 30, None) == -1
    assert L.qlora_mlp_fwd(ctypes.byref(g), ctypes.byref(u), ctypes.byref(d), dummy, 64, ptrs, ptrs, 8, 16.0,
                           ctypes.c_void_p(4098), None, None, ws, 1 << 30, None) == -1  # Y misaligned
    assert L.qlora_mlp_bwd(ctypes.byref(g), ctypes.byref(u), ctypes.byref(d), dummy, dummy, 64, ptrs, ptrs, 8, 16.0,
                           None, None, dummy, ptrs, VP(dummy, None, dummy), ws, 1 << 30, None) == -1
    assert L.qlora_mlp_bwd(ctypes.byref(g), ctypes.byref(u), ctypes.byref(d), dummy, ctypes.c_void_p(4098), 64, ptrs,
                           ptrs, 8, 16.0, None, None, dummy, ptrs, ptrs, ws, 1 << 30, None) == -1  # dY misaligned
    # G and U saved together or not at all
    assert L.qlora_mlp_bwd(ctypes.byref(g), ctypes.byref(u), ctypes.byref(d), dummy, dummy, 64, ptrs, ptrs, 8, 16.0,
                           dummy, None, dummy, ptrs, ptrs, ws, 1 << 30, None) == -1
    assert L.qlora_mlp_bwd(ctypes.byref(g), ctypes.byref(u), ctypes.byref(d), dummy, dummy, 64, ptrs, ptrs, 8, 16.0,
                           None, None, dummy, ptrs, ptrs, ws, 16, None) == -5


def test_grouped_workspace_covers_every_single_call():
    """A group's workspace also holds each linear's own forward (the path taken when the
    group does not run as one launch) and, for the one-launch case, the group's partials."""
    from bit_nf4_quantized_dq_amd import QuantizedWeight
    import torch

    z = torch.zeros(16, dtype=torch.uint8)  # host buffers: only the sizes are read

    def fake(d_out, d_in):
        return QuantizedWeight(z, z, z.view(torch.float32), z.view(torch.float32)[:1], d_out, d_in)

    for dims, M, r in [([8192, 1024, 1024], 1, 16), ([28672, 28672], 1, 16), ([4096, 4096], 16, 128),
                       ([1008, 512], 4, 8), ([4096, 1024, 1024], 4096, 16)]:
        qs = [fake(d, 8192 if dims[0] > 5000 else 4096) for d in dims]
        need = B.workspace_size_multi(qs, M, r)
        for q in qs:
            assert need >= B.workspace_size(B.OP_FWD, M, q.d_out, q.d_in, r)
        if M <= 16 and all(d % 256 == 0 for d in dims) and sum(dims) * qs[0].d_in >= (32 << 20):
            assert need >= 4 * M * sum(dims)  # at least one split of FP32 partials


def test_workspace_sizes_are_sane():
    for M in (1, 16, 17, 4096):
        for op in (B.OP_FWD, B.OP_BWD):
            n = B.workspace_size(op, M, 4096, 4096, 16)
            assert 256 <= n < (64 << 20) + 64 * M * 16 * 4
    assert B.workspace_size(B.OP_QUANTIZE, 1, 4096, 4096, 1) >= 4096 * 4096 // 64 * 4


def test_weight_stream_plan_without_a_fitting_split():
    """A shape at the edge of the limits for which no split of the weight stream fits its
    staging limits (1024 rows of 2^22 weights): the plan reports none, and the other path
    serves it (the plan once divided by the empty split count)."""
    for M in (1, 4, 16):
        for r in (8, 64, 128):
            assert B.workspace_size(B.OP_FWD, M, 1024, 1 << 22, r) > 0
            assert B.workspace_size(B.OP_FWD, M, 1 << 22, 1024, r) > 0


def test_strerror_covers_every_status(L):
    for s in range(0, -8, -1):
        assert B._strerror(s) not in ("?", "unknown status")


@pytest.mark.parametrize("name", ["nf4", "int4", "fp4"])
def test_codebooks_equal_oracle_bit_for_bit(name):
    lib_levels = np.array(B.codebook(name), dtype=np.float32)
    assert np.array_equal(lib_levels.view(np.uint32), O.codebook(name).view(np.uint32))


@pytest.mark.parametrize("dq", ["e4m3", "e5m2", "int8", "none"])
def test_format_sizes_match_oracle(dq):
    a, b, c = B.quant_sizes(1024, 4096, dq)
    sz = O.quant_sizes(1024, 4096, dq)
    assert (a, b, c) == (sz["codes"], sz["code8"], sz["c2s"])


def test_workspace_grows_for_decode_once_formats():
    """Only E4M3 constants are decoded inside the small-M kernels; other formats need the
    BF16 weight copy in the workspace at every M."""
    base = B.workspace_size(B.OP_FWD, 1, 4096, 4096, 16, "e4m3")
    for dq in ("e5m2", "int8", "none"):
        assert B.workspace_size(B.OP_FWD, 1, 4096, 4096, 16, dq) >= 2 * 4096 * 4096 > base


# ------------------------------------------------------------------ binding checks (no GPU)


def _cpu_weight(d_out=256, d_in=256):
    import torch

    from bit_nf4_quantized_dq_amd import QuantizedWeight

    nc, n8, n2 = B.quant_sizes(d_out, d_in)
    return QuantizedWeight(torch.zeros(nc, dtype=torch.uint8), torch.zeros(n8, dtype=torch.uint8),
                           torch.zeros(n2 // 4), torch.zeros(1), d_out, d_in)


def test_binding_rejects_mis_shaped_operands_before_any_call():
    """The C ABI sees raw pointers only, so the binding checks every tensor's shape against the
    weight, M and r first: a wrong shape is reported by name (CPU tensors: every shape and
    dtype is checked before the device), and right shapes get as far as the device check."""
    import torch

    bf = torch.bfloat16
    q = _cpu_weight(256, 512)
    M, r = 4, 8
    X, A, Bm = torch.zeros(M, 512, dtype=bf), torch.zeros(r, 512, dtype=bf), torch.zeros(256, r, dtype=bf)
    dY = torch.zeros(M, 256, dtype=bf)
    cases = [
        (lambda: B.linear_fwd(q, torch.zeros(M, 256, dtype=bf), A, Bm, 16.0), "X"),
        (lambda: B.linear_fwd(q, X, torch.zeros(r, 256, dtype=bf), Bm, 16.0), "A"),
        (lambda: B.linear_fwd(q, X, A, torch.zeros(512, r, dtype=bf), 16.0), "B"),
        (lambda: B.linear_fwd(q, X, A, torch.zeros(256, r + 1, dtype=bf), 16.0), "B"),
        (lambda: B.linear_fwd(q, X, A, Bm, 16.0, Y=torch.zeros(M, 512, dtype=bf)), "Y"),
        (lambda: B.linear_fwd(q, X, A, Bm, 16.0, T_save=torch.zeros(M, r + 1, dtype=bf)), "T_save"),
        (lambda: B.linear_fwd(q, X.float(), A, Bm, 16.0), "X"),
        (lambda: B.linear_bwd(q, X, torch.zeros(M, 512, dtype=bf), A, Bm, 16.0), "dY"),
        (lambda: B.linear_bwd(q, X, dY, A, Bm, 16.0, T_saved=torch.zeros(M + 1, r, dtype=bf)), "T_saved"),
        (lambda: B.linear_bwd(q, X, dY, A, Bm, 16.0, dX=torch.zeros(M, 256, dtype=bf)), "dX"),
        (lambda: B.linear_bwd(q, X, dY, A, Bm, 16.0, dA=torch.zeros(r, 256, dtype=bf)), "dA"),
        (lambda: B.linear_bwd(q, X, dY, A, Bm, 16.0, dB=torch.zeros(r, 256, dtype=bf)), "dB"),
        (lambda: B.merge(q, A, Bm, 16.0, out=torch.zeros(512, 256, dtype=bf)), "out"),
        (lambda: B.dequantize(q, out=torch.zeros(256, 256, dtype=bf)), "out"),
        (lambda: B.linear_fwd(_cpu_weight(256, 512).__class__(q.codes[:-1], q.code8, q.c2s, q.mu, 256, 512), X, A, Bm,
                              16.0), "weight.codes"),
        (lambda: B.linear_fwd_multi([q, q], X, [A, A], [Bm, torch.zeros(256, r - 1, dtype=bf)], 16.0), "B[1]"),
        (lambda: B.linear_fwd_multi([q, q], X, [A], [Bm, Bm], 16.0), "one A"),
    ]
    for fn, name in cases:
        with pytest.raises(ValueError, match=re.escape(name)):
            fn()
    # correctly shaped host tensors pass the shape checks and stop at the device check
    with pytest.raises(ValueError, match="CUDA"):
        B.linear_fwd(q, X, A, Bm, 16.0)
    with pytest.raises(ValueError, match="CUDA"):
        B.linear_bwd(q, X, dY, A, Bm, 16.0)


def test_binding_rejects_mis_shaped_mlp_operands():
    import torch

    bf = torch.bfloat16
    d, f, M, r = 256, 512, 4, 8
    qs = [_cpu_weight(f, d), _cpu_weight(f, d), _cpu_weight(d, f)]
    As = [torch.zeros(r, d, dtype=bf), torch.zeros(r, d, dtype=bf), torch.zeros(r, f, dtype=bf)]
    Bs = [torch.zeros(f, r, dtype=bf), torch.zeros(f, r, dtype=bf), torch.zeros(d, r, dtype=bf)]
    X, dY = torch.zeros(M, d, dtype=bf), torch.zeros(M, d, dtype=bf)
    with pytest.raises(ValueError, match=re.escape("A[2]")):
        B.mlp_fwd(qs, X, As[:2] + [torch.zeros(r, d, dtype=bf)], Bs, 16.0)
    with pytest.raises(ValueError, match="G_save"):
        B.mlp_fwd(qs, X, As, Bs, 16.0, G_save=torch.zeros(M, d, dtype=bf))
    with pytest.raises(ValueError, match="U_saved"):
        B.mlp_bwd(qs, X, dY, As, Bs, 16.0, G_saved=torch.zeros(M, f, dtype=bf), U_saved=torch.zeros(M, f))
    with pytest.raises(ValueError, match="both"):
        B.mlp_bwd(qs, X, dY, As, Bs, 16.0, G_saved=torch.zeros(M, f, dtype=bf))
    with pytest.raises(ValueError, match="CUDA"):
        B.mlp_bwd(qs, X, dY, As, Bs, 16.0)
