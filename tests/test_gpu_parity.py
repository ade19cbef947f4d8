"""GPU parity: the HIP library (through its C ABI) against the CPU oracle on identical seeded
inputs.  Encode/decode outputs must match bit for bit; forward/backward outputs must be
within a normwise relative error of 1e-2: max|got - ref| / max|ref| <= 1e-2 per tensor."""

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


def _assert_quant_equal(q, oq):
    assert np.array_equal(_np(q.codes), oq["packed"].reshape(-1)), "packed codes"
    assert np.array_equal(_np(q.code8), oq["code8"]), "code8"
    assert np.array_equal(_np(q.c2s).view(np.uint32), oq["c2s"].view(np.uint32)), "c2s"
    assert _np(q.mu).view(np.uint32)[0] == np.float32(oq["mu"]).view(np.uint32), "mu"


def _case(cfg, d_out, d_in, M, r, std, idx=0):
    c = I.linear_case(cfg, idx, d_out, d_in, M, r, std)
    return c


# ---------------------------------------------------------------- encoders

def test_e4m3_encoder_matches_oracle(gpu_lib):
    from bit_nf4_quantized_dq_amd import e4m3_encode

    vals = O.e4m3_value(np.arange(0, 0x7F)).astype(np.float64)
    mids = 0.5 * (vals[:-1] + vals[1:])
    pts = []
    for m in np.concatenate([vals, mids]):
        f = np.float32(m)
        pts += [f, np.nextafter(f, np.float32(0)), np.nextafter(f, np.float32(1e9))]
    rng = np.random.default_rng(0)
    pts = np.array(pts, dtype=np.float32)
    pts = np.concatenate([pts, -pts, rng.uniform(-449, 449, 200000).astype(np.float32),
                          np.array([0.0, -0.0, 1e-30, -1e-30, 448.0, -448.0], np.float32)])
    got = _np(e4m3_encode(torch.from_numpy(pts).cuda()))
    assert np.array_equal(got, O.e4m3_encode(pts))


# ---------------------------------------------------------------- quantize / dequantize

QSHAPES = [(1, 256, 256, 0.02), (2, 4096, 4096, 0.02), (9, 272, 320, 0.02), (9, 16, 64, 0.02), (4, 1024, 4096, 0.02)]


@pytest.mark.parametrize("cfg,d_out,d_in,std", QSHAPES)
def test_quantize_and_dequantize_bit_exact(gpu_lib, cfg, d_out, d_in, std):
    from bit_nf4_quantized_dq_amd import dequantize, quantize

    W = I.weight(cfg, 0, d_out, d_in, std)
    oq = O.quantize(W.numpy())
    q = quantize(W.cuda())
    torch.cuda.synchronize()
    _assert_quant_equal(q, oq)
    w = dequantize(q)
    torch.cuda.synchronize()
    assert np.array_equal(_np(w.view(torch.int16)).view(np.uint16), O.dequantize_bf16_bits(oq))


def test_quantize_special_values(gpu_lib):
    """Zero blocks, exact zeros, a lone outlier, FP32 subnormals, a huge block and exact
    NF4 multiples in one tensor."""
    from bit_nf4_quantized_dq_amd import dequantize, quantize

    rng = np.random.default_rng(3)
    W = (rng.standard_normal((64, 512)) * 0.02).astype(np.float32)
    W[0, :64] = 0.0
    W[1, 5] = 0.0
    W[2, 100] = 40.0
    W[3, :64] = (rng.standard_normal(64) * 1e-40).astype(np.float32)  # subnormal block
    W[4, 64:128] = np.float32(1e30) * rng.standard_normal(64).astype(np.float32)
    W[5, :64] = O.nf4_codebook()[rng.integers(0, 16, 64)] * np.float32(0.25)
    W[6, 0:64] = -W[6, 0:64]
    oq = O.quantize(W)
    q = quantize(torch.from_numpy(W).cuda())
    torch.cuda.synchronize()
    _assert_quant_equal(q, oq)
    w = dequantize(q)
    assert np.array_equal(_np(w.view(torch.int16)).view(np.uint16), O.dequantize_bf16_bits(oq))


def test_roundtrip_special_case_gpu(gpu_lib):
    from bit_nf4_quantized_dq_amd import dequantize, quantize

    q_tab = O.nf4_codebook()
    rng = np.random.default_rng(5)
    k = rng.integers(0, 16, size=(128, 1024))
    k[:, ::64] = 0
    W = (q_tab[k] * np.float32(2.0**-5)).astype(np.float32)
    q = quantize(torch.from_numpy(W).cuda())
    w = dequantize(q)
    exp = torch.from_numpy(W).to(torch.bfloat16)
    assert torch.equal(w.cpu().view(torch.int16), exp.view(torch.int16))


def test_quantize_rejects_nonfinite(gpu_lib):
    from bit_nf4_quantized_dq_amd import QLoRAError, quantize

    W = torch.randn(64, 256)
    W[7, 9] = float("nan")
    with pytest.raises(QLoRAError) as e:
        quantize(W.cuda())
    assert e.value.status == -4
    W[7, 9] = float("inf")
    with pytest.raises(QLoRAError):
        quantize(W.cuda())


# ---------------------------------------------------------------- forward / backward


def _run(c, alpha, r, zero_w=False, t_saved=True, need_dx=True):
    from bit_nf4_quantized_dq_amd import linear_bwd, linear_fwd, quantize

    W = torch.zeros_like(c["W"]) if zero_w else c["W"]
    oq = O.quantize(W.numpy())
    what = O.dequantize_f64(oq)
    X, A, Bm, dY = (c[k] for k in ("X", "A", "B", "dY"))
    Xd, Ad, Bd, dYd = (t.cuda() for t in (X, A, Bm, dY))
    q = quantize(W.cuda())
    M = X.shape[0]
    T = torch.empty(M, r, dtype=torch.bfloat16, device="cuda")
    Y = linear_fwd(q, Xd, Ad, Bd, alpha, T_save=T)
    dX, dA, dB = linear_bwd(q, Xd, dYd, Ad, Bd, alpha, T_saved=T if t_saved else None, need_dX=need_dx)
    torch.cuda.synchronize()
    Yr, Tr = O.lora_fwd(what, _f64(X), _f64(A), _f64(Bm), alpha, r)
    dXr, dAr, dBr = O.lora_bwd(what, _f64(X), _f64(dY), _f64(A), _f64(Bm), alpha, r)
    return dict(Y=(_f64(Y), Yr), T=(_f64(T), Tr), dA=(_f64(dA), dAr), dB=(_f64(dB), dBr),
                dX=(_f64(dX) if need_dx else None, dXr))


FB_CASES = [
    # cfg, d_out, d_in, M, r, alpha
    (1, 256, 256, 4, 8, 16.0),
    (9, 272, 320, 1, 8, 16.0),
    (9, 272, 320, 16, 16, 32.0),
    (9, 272, 320, 17, 16, 32.0),
    (9, 272, 320, 300, 16, 32.0),
    (9, 512, 1024, 777, 24, 48.0),
    (9, 1040, 192, 513, 8, 16.0),
    (9, 64, 2048, 100, 128, 256.0),
    (9, 2048, 64, 40, 3, 6.0),
    # M <= 16: more adapter ranks and reduction splits
    (9, 528, 192, 3, 40, 80.0),     # r not a multiple of 8
    (9, 64, 2048, 2, 128, 256.0),   # the largest rank
    (9, 1040, 4096, 1, 5, 10.0),    # ragged rank tile, a deep reduction split
    (9, 16, 64, 16, 16, 32.0),      # a single row group, a single block per row
    # M >= 1024: decoded weight copy + plain BF16 GEMM
    (9, 272, 320, 1100, 16, 32.0),  # ragged M and N; the dX reduction (over N) ends mid-step
    (9, 528, 192, 1025, 40, 80.0),  # two adapter slices, r not a multiple of 8
    (9, 64, 2048, 1024, 128, 256.0),  # four adapter slices, one feature tile
    # rank 1 (the smallest adapter) on each path
    (9, 272, 320, 4, 1, 2.0),
    (9, 272, 320, 300, 1, 2.0),
    (9, 272, 320, 1100, 1, 2.0),
]


@pytest.mark.parametrize("cfg,d_out,d_in,M,r,alpha", FB_CASES)
def test_fwd_bwd_parity(gpu_lib, cfg, d_out, d_in, M, r, alpha):
    c = _case(cfg, d_out, d_in, M, r, 0.02)
    res = _run(c, alpha, r)
    for k, (got, ref) in res.items():
        e = normwise(got, ref)
        assert e <= TOL, (k, e)


@pytest.mark.parametrize("M", [1, 16, 300, 1100])
def test_lora_path_in_isolation(gpu_lib, M):
    """W = 0: Y = s T B^T and dX = s G A exactly as the adapter branch alone."""
    c = _case(9, 272, 320, M, 16, 0.02)
    res = _run(c, 32.0, 16, zero_w=True, t_saved=False)
    for k in ("Y", "dX", "dA", "dB"):
        got, ref = res[k]
        assert np.max(np.abs(ref)) > 0
        assert normwise(got, ref) <= TOL, k


@pytest.mark.parametrize("M", [33, 1030])
def test_alpha_zero_is_base_only(gpu_lib, M):
    c = _case(9, 272, 320, M, 8, 0.02)
    res = _run(c, 0.0, 8, need_dx=True)
    for k in ("Y", "dX"):
        got, ref = res[k]
        assert normwise(got, ref) <= TOL
    assert np.all(res["dA"][0] == 0) and np.all(res["dB"][0] == 0)


def test_no_dx_requested(gpu_lib):
    c = _case(9, 272, 320, 64, 8, 0.02)
    res = _run(c, 16.0, 8, need_dx=False)
    assert res["dX"][0] is None
    for k in ("dA", "dB"):
        assert normwise(*res[k]) <= TOL


def test_weights_read_only_and_deterministic(gpu_lib):
    from bit_nf4_quantized_dq_amd import linear_bwd, linear_fwd, quantize

    c = _case(9, 512, 512, 300, 16, 0.02)
    q = quantize(c["W"].cuda())
    before = [t.clone() for t in (q.codes, q.code8, q.c2s, q.mu)]
    X, A, Bm, dY = (c[k].cuda() for k in ("X", "A", "B", "dY"))
    outs = []
    for _ in range(2):
        Y = linear_fwd(q, X, A, Bm, 32.0)
        dX, dA, dB = linear_bwd(q, X, dY, A, Bm, 32.0)
        Ys = linear_fwd(q, X[:8].contiguous(), A, Bm, 32.0)
        outs.append([t.clone() for t in (Y, dX, dA, dB, Ys)])
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    for a, b in zip(before, (q.codes, q.code8, q.c2s, q.mu)):
        assert torch.equal(a, b)


# ---------------------------------------------------------------- the named workloads


def test_config2_weight_stream_4096(gpu_lib):
    """4096x4096 at M=1 and M=16, forward only."""
    for M in (1, 16):
        c = _case(2, 4096, 4096, M, 16, 0.02)
        from bit_nf4_quantized_dq_amd import linear_fwd, quantize

        q = quantize(c["W"].cuda())
        oq = O.quantize(c["W"].numpy())
        _assert_quant_equal(q, oq)
        Y = linear_fwd(q, c["X"].cuda(), c["A"].cuda(), c["B"].cuda(), 32.0)
        Yr, _ = O.lora_fwd(O.dequantize_f64(oq), _f64(c["X"]), _f64(c["A"]), _f64(c["B"]), 32.0, 16)
        assert normwise(_f64(Y), Yr) <= TOL


def test_config3_train_step_4096(gpu_lib):
    """4096x4096 at M=4096: forward and backward against the full FP64 oracle."""
    c = _case(3, 4096, 4096, 4096, 16, 0.02)
    res = _run(c, 32.0, 16)
    for k, (got, ref) in res.items():
        assert normwise(got, ref) <= TOL, k


@pytest.mark.parametrize("idx", range(7))
def test_config4_llama3_8b_layer_sampled(gpu_lib, idx):
    """Llama-3-8B layer linears at M=8192: encode/decode checked on sampled blocks;
    outputs checked on sampled tokens and features; dA/dB in full."""
    from bit_nf4_quantized_dq_amd import dequantize, linear_bwd, linear_fwd, quantize

    shp = I.LLAMA3_8B_LAYER[idx]
    N, K, M, r, alpha = shp.d_out, shp.d_in, 8192, 16, 32.0
    c = I.linear_case(4, idx, N, K, M, r, 0.02)
    rng = np.random.default_rng(idx)
    n_s = np.sort(rng.choice(N, 48, replace=False))
    kb_s = int(rng.integers(0, K // 64))
    m_s = np.sort(rng.choice(M, 48, replace=False))
    mask = np.zeros((N, K // 64), bool)
    mask[n_s, :] = True
    mask[:, kb_s] = True
    oq = O.quantize(c["W"].numpy(), blocks=mask)
    what = O.dequantize_f64(oq)  # NaN outside the sampled blocks
    q = quantize(c["W"].cuda())
    X, A, Bm, dY = (c[k].cuda() for k in ("X", "A", "B", "dY"))
    T = torch.empty(M, r, dtype=torch.bfloat16, device="cuda")
    Y = linear_fwd(q, X, A, Bm, alpha, T_save=T)
    dX, dA, dB = linear_bwd(q, X, dY, A, Bm, alpha, T_saved=T)
    wq = dequantize(q)
    torch.cuda.synchronize()
    # encode/decode on the sampled blocks
    assert np.array_equal(_np(q.code8), oq["code8"]) and np.array_equal(_np(q.c2s), oq["c2s"])
    assert _np(q.mu)[0] == oq["mu"]
    gw = _np(wq.view(torch.int16)).view(np.uint16)
    ow = O.dequantize_bf16_bits(oq)
    sel = np.repeat(mask, 64, axis=1)
    assert np.array_equal(gw[sel], ow[sel])
    s = alpha / r
    Xf, Af, Bf, dYf = _f64(c["X"]), _f64(c["A"]), _f64(c["B"]), _f64(c["dY"])
    T_ref = Xf @ Af.T
    G_ref = dYf @ Bf
    # forward on sampled (token, feature) pairs
    Y_ref = Xf[m_s] @ what[n_s].T + s * T_ref[m_s] @ Bf[n_s].T
    assert normwise(_f64(Y)[np.ix_(m_s, n_s)], Y_ref) <= TOL
    # dX on sampled tokens, one column block
    cols = slice(64 * kb_s, 64 * kb_s + 64)
    dX_ref = dYf[m_s] @ what[:, cols] + s * G_ref[m_s] @ Af[:, cols]
    assert normwise(_f64(dX)[m_s][:, cols], dX_ref) <= TOL
    assert normwise(_f64(dA), s * G_ref.T @ Xf) <= TOL
    assert normwise(_f64(dB), s * dYf.T @ T_ref) <= TOL
    assert normwise(_f64(T), T_ref) <= TOL


# d_out * d_in >= 32M with d_in a multiple of 256: the large-weight stream kernel
@pytest.mark.parametrize("M,r", [(1, 8), (7, 24), (16, 32), (3, 16)])
def test_weight_stream_full_chunk_adapter_first(gpu_lib, M, r):
    """4096x4096 at M <= 16 splits d_in into 8 ranges of one full chunk, where the adapter part
    runs before the weight codes are staged: Y and T in full against the oracle."""
    from bit_nf4_quantized_dq_amd import linear_fwd, quantize

    N = K = 4096
    alpha = 2.0 * r
    print(f"full-chunk 4096x4096 M={M} r={r}", flush=True)
    c = _case(14, N, K, M, r, 0.02, idx=M + r)
    oq = O.quantize(c["W"].numpy())
    what = O.bf16_bits_to_f32(O.dequantize_bf16_bits(oq)).astype(np.float64)
    q = quantize(c["W"].cuda())
    T = torch.empty(M, r, dtype=torch.bfloat16, device="cuda")
    Y = linear_fwd(q, c["X"].cuda(), c["A"].cuda(), c["B"].cuda(), alpha, T_save=T)
    torch.cuda.synchronize()
    Xf, Af, Bf = _f64(c["X"]), _f64(c["A"]), _f64(c["B"])
    T_ref = Xf @ Af.T
    assert normwise(_f64(Y), Xf @ what.T + (alpha / r) * T_ref @ Bf.T) <= TOL
    assert normwise(_f64(T), T_ref) <= TOL


ROWS_CASES = [
    # d_out, d_in, M, r: whole rows per workgroup (M <= 4, at least 4096 rows, d_in 2048 or 4096)
    (4096, 2048, 3, 8),    # the shorter reduction
    (6144, 4096, 2, 64),   # 384 row groups, 64 T workgroups
    (4096, 4096, 1, 40),   # a rank that ends inside a 32-wide step
    (5120, 4096, 4, 24),
    (4096, 4096, 4, 16),
    (4096, 2048, 4, 128),  # rank 128 (the largest): the handed-over words fill the 512 KiB head
]


@pytest.mark.parametrize("N,K,M,r", ROWS_CASES)
def test_weight_stream_whole_rows(gpu_lib, N, K, M, r):
    """M <= 16 with whole rows per workgroup and T handed over through the workspace head:
    Y and T in full against the oracle, over three calls on one workspace (the handed-over
    words are cleared by each call)."""
    from bit_nf4_quantized_dq_amd import OP_FWD, linear_fwd, new_workspace, quantize, workspace_size

    print(f"rows {N}x{K} M={M} r={r}", flush=True)
    alpha = 2.0 * r
    c = _case(18, N, K, M, r, 0.02, idx=M + r)
    oq = O.quantize(c["W"].numpy())
    what = O.bf16_bits_to_f32(O.dequantize_bf16_bits(oq)).astype(np.float64)
    q = quantize(c["W"].cuda())
    ws = new_workspace(workspace_size(OP_FWD, M, N, K, r), "cuda")
    X, A, Bm = c["X"].cuda(), c["A"].cuda(), c["B"].cuda()
    Xf, Af, Bf = _f64(c["X"]), _f64(c["A"]), _f64(c["B"])
    T_ref = Xf @ Af.T
    Y_ref = Xf @ what.T + (alpha / r) * T_ref @ Bf.T
    first = None
    for call in range(3):
        T = torch.empty(M, r, dtype=torch.bfloat16, device="cuda")
        Y = linear_fwd(q, X, A, Bm, alpha, T_save=T, ws=ws)
        torch.cuda.synchronize()
        assert normwise(_f64(Y), Y_ref) <= TOL, call
        assert normwise(_f64(T), T_ref) <= TOL, call
        if first is None:
            first = Y.clone()
        assert torch.equal(Y.view(torch.int16), first.view(torch.int16)), call
    assert int(ws[:524288].view(torch.int32).abs().sum()) == 0, "the counter head is left zero"


def test_weight_stream_whole_rows_token_independence(gpu_lib):
    """Each token's output of the whole-row kernel depends on that token alone: a 4-token
    call equals 4 one-token calls, and a 3-token call equals a 2-token call plus a 1-token
    call, bit for bit, Y and T."""
    from bit_nf4_quantized_dq_amd import linear_fwd, quantize

    N, K, r = 4096, 4096, 16
    c = _case(19, N, K, 4, r, 0.02, idx=3)
    q = quantize(c["W"].cuda())
    X, A, Bm = c["X"].cuda(), c["A"].cuda(), c["B"].cuda()

    def fwd(rows):
        T = torch.empty(rows.shape[0], r, dtype=torch.bfloat16, device="cuda")
        Y = linear_fwd(q, rows.contiguous(), A, Bm, 32.0, T_save=T)
        return Y.clone(), T.clone()

    Y4, T4 = fwd(X)
    parts = [fwd(X[m:m + 1]) for m in range(4)]
    Y3, T3 = fwd(X[:3])
    Y2, T2 = fwd(X[:2])
    torch.cuda.synchronize()
    bits = lambda t: t.view(torch.int16)
    assert torch.equal(bits(Y4), bits(torch.cat([p[0] for p in parts])))
    assert torch.equal(bits(T4), bits(torch.cat([p[1] for p in parts])))
    assert torch.equal(bits(Y3), bits(torch.cat([Y2, parts[2][0]])))
    assert torch.equal(bits(T3), bits(torch.cat([T2, parts[2][1]])))


STREAM_CASES = [
    # d_out, d_in, M, r
    (8192, 4096, 1, 16),
    (8192 + 160, 4096, 3, 40),  # a partial row group; B ranks past 32 read element by element
    (4352, 8192, 16, 128),      # M = 16 and the largest rank
    (12288, 4096, 2, 8),
    (8192, 4096, 1, 40),        # M = 1: T handed over by producer workgroups, B rows read by element
    (1024, 40960, 1, 16),       # M = 1 with a reduction past 32768: T formed in the loop
]


@pytest.mark.parametrize("N,K,M,r", STREAM_CASES)
def test_weight_stream_large_shapes(gpu_lib, N, K, M, r):
    """Large weights at M <= 16: Y on sampled features (every row group boundary and the last
    rows included) against the oracle on those rows; the saved T in full."""
    from bit_nf4_quantized_dq_amd import linear_fwd, quantize

    print(f"stream {N}x{K} M={M} r={r}", flush=True)
    alpha = 2.0 * r
    c = _case(9, N, K, M, r, 0.02, idx=40 + M)
    rng = np.random.default_rng(N + K + M + r)
    n_s = np.unique(np.concatenate([rng.choice(N, 40, replace=False), np.arange(0, N, 256)[:8], [255, 256, N - 1]]))
    mask = np.zeros((N, K // 64), bool)
    mask[n_s, :] = True
    oq = O.quantize(c["W"].numpy(), blocks=mask)
    what = O.bf16_bits_to_f32(O.dequantize_bf16_bits(oq)[n_s]).astype(np.float64)
    q = quantize(c["W"].cuda())
    T = torch.empty(M, r, dtype=torch.bfloat16, device="cuda")
    Y = linear_fwd(q, c["X"].cuda(), c["A"].cuda(), c["B"].cuda(), alpha, T_save=T)
    torch.cuda.synchronize()
    Xf, Af, Bf = _f64(c["X"]), _f64(c["A"]), _f64(c["B"])
    T_ref = Xf @ Af.T
    Y_ref = Xf @ what.T + (alpha / r) * T_ref @ Bf[n_s].T
    assert normwise(_f64(Y)[:, n_s], Y_ref) <= TOL
    assert normwise(_f64(T), T_ref) <= TOL


def test_weight_stream_graph_replay(gpu_lib):
    """The M <= 16 path captured in a HIP graph and replayed with new inputs in between:
    every replay equals an eager call on the same inputs (the split-K arrival counters
    carry no per-call host state)."""
    from bit_nf4_quantized_dq_amd import QuantizedWeight, linear_fwd, new_workspace, quantize, workspace_size, OP_FWD

    dev = torch.device("cuda")
    shapes = [(1040, 4096, 1, 16), (272, 320, 16, 16), (4096, 4096, 16, 16), (8192, 4096, 1, 16)]
    cases = []
    for i, (N, K, M, r) in enumerate(shapes):
        c = _case(9, N, K, M, r, 0.02, idx=10 + i)
        q = quantize(c["W"].to(dev))
        X = c["X"].to(dev)
        A, B = c["A"].to(dev), c["B"].to(dev)
        Y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        ws = new_workspace(workspace_size(OP_FWD, M, N, K, r), dev)
        cases.append((q, X, A, B, Y, ws))
    for q, X, A, B, Y, ws in cases:  # warm-up outside the capture
        linear_fwd(q, X, A, B, 32.0, Y=Y, ws=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            for q, X, A, B, Y, ws in cases:
                linear_fwd(q, X, A, B, 32.0, Y=Y, ws=ws)
    torch.cuda.synchronize()
    gen = torch.Generator(device="cpu").manual_seed(77)
    for rep in range(4):
        for q, X, A, B, Y, ws in cases:
            X.copy_(torch.randn(X.shape, generator=gen).to(torch.bfloat16))
            A.copy_((torch.randn(A.shape, generator=gen) * 0.02).to(torch.bfloat16))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [Y.clone() for *_, Y, _ in cases]
        for (q, X, A, B, Y, ws), yg in zip(cases, got):
            ye = linear_fwd(q, X, A, B, 32.0)
            torch.cuda.synchronize()
            assert torch.equal(ye.view(torch.int16), yg.view(torch.int16)), f"replay {rep}"


@pytest.mark.parametrize("N,K,M", [
    (528, 2112, 1100),   # 3 x 5 tiles, ragged edges; 66 reduction steps over 4 splits (17, 17, 17, 15)
    (1024, 8192, 2048),  # a k/v projection of the 70B-class model: 32 tiles, 8 splits
])
def test_split_reduction_gemm(gpu_lib, N, K, M):
    """Forward at M >= 1024 through the decoded copy, on a product with few tiles, so the BF16
    GEMM splits its reduction over several workgroups and sums the FP32 partials in a second
    launch: every output against the oracle (the second shape on sampled rows)."""
    from bit_nf4_quantized_dq_amd import linear_fwd, quantize

    r, alpha = 16, 32.0
    print(f"split gemm {N}x{K} M={M}", flush=True)
    c = _case(13, N, K, M, r, 0.02, idx=N % 97)
    rng = np.random.default_rng(N + K + M)
    n_s = np.arange(N) if N * K <= (4 << 20) else np.sort(rng.choice(N, 48, replace=False))
    mask = np.zeros((N, K // 64), bool)
    mask[n_s, :] = True
    oq = O.quantize(c["W"].numpy(), blocks=mask)
    what = O.bf16_bits_to_f32(O.dequantize_bf16_bits(oq)[n_s]).astype(np.float64)
    q = quantize(c["W"].cuda())
    T = torch.empty(M, r, dtype=torch.bfloat16, device="cuda")
    Y = linear_fwd(q, c["X"].cuda(), c["A"].cuda(), c["B"].cuda(), alpha, T_save=T)
    torch.cuda.synchronize()
    Xf, Af, Bf = _f64(c["X"]), _f64(c["A"]), _f64(c["B"])
    T_ref = Xf @ Af.T
    Y_ref = Xf @ what.T + (alpha / r) * T_ref @ Bf[n_s].T
    assert normwise(_f64(Y)[:, n_s], Y_ref) <= TOL
    assert normwise(_f64(T), T_ref) <= TOL


@pytest.mark.parametrize("idx", [0, 2, 4, 6])
def test_config5_70b_shapes_sampled(gpu_lib, idx):
    """70B-class layer linears (layer 79 of the seed rule), forward at M = 1 (weight stream)
    and M = 2048 (decoded copy + BF16 GEMM): encode/decode on sampled blocks, outputs on
    sampled (token, feature) pairs."""
    from bit_nf4_quantized_dq_amd import dequantize, linear_fwd, quantize

    shp = I.SEVENTY_B_LAYER[idx]
    N, K, r, alpha, layer = shp.d_out, shp.d_in, 16, 32.0, 79
    print(f"70B {shp.name} {N}x{K}", flush=True)
    W = I.weight(5, idx, N, K, 0.015, layer)
    rng = np.random.default_rng(100 + idx)
    n_s = np.sort(rng.choice(N, 32, replace=False))
    kb_s = int(rng.integers(0, K // 64))
    mask = np.zeros((N, K // 64), bool)
    mask[n_s, :] = True
    mask[:, kb_s] = True
    oq = O.quantize(W.numpy(), blocks=mask)
    q = quantize(W.cuda())
    wq = dequantize(q)
    torch.cuda.synchronize()
    assert np.array_equal(_np(q.code8), oq["code8"]) and np.array_equal(_np(q.c2s), oq["c2s"])
    assert _np(q.mu)[0] == oq["mu"]
    sel = np.repeat(mask, 64, axis=1)
    ob = O.dequantize_bf16_bits(oq)
    assert np.array_equal(_np(wq.view(torch.int16)).view(np.uint16)[sel], ob[sel])
    del wq
    what = O.bf16_bits_to_f32(ob[n_s]).astype(np.float64)
    del ob, sel
    A = I.lora_A(5, idx, r, K, layer)
    Bm = I.lora_B(5, idx, N, r, layer)
    Af, Bf = _f64(A), _f64(Bm)
    for M in (1, 2048):
        X = I.activations(5, idx, M, K, layer)
        m_s = np.arange(M) if M == 1 else np.sort(rng.choice(M, 32, replace=False))
        Y = linear_fwd(q, X.cuda(), A.cuda(), Bm.cuda(), alpha)
        torch.cuda.synchronize()
        Xf = _f64(X)[m_s]
        Y_ref = Xf @ what.T + (alpha / r) * (Xf @ Af.T) @ Bf[n_s].T
        assert normwise(_f64(Y)[np.ix_(m_s, n_s)], Y_ref) <= TOL, M
