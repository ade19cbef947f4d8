"""ctypes binding of include/qlora.h.  Argument marshalling only: torch tensors provide
device memory (``data_ptr``) and the stream (``cuda_stream``); every step of the method runs
in the HIP library."""

from __future__ import annotations

import ctypes
import dataclasses
import functools
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libqlora_nf4.so")

OP_QUANTIZE, OP_FWD, OP_BWD = 0, 1, 2
CODEBOOKS = {"nf4": 0, "int4": 1, "fp4": 2}
DQ_FORMATS = {"e4m3": 0, "e5m2": 1, "int8": 2, "none": 3}
KERNEL_IDS = {
    "quant_pass1": 0,
    "quant_pass2": 1,
    "dequant": 2,
    "gemv_fwd": 3,
    "gemm_fwd": 4,
    "gemm_dx": 5,
    "lora_down": 6,
    "lora_grad": 7,
    "dequant_t": 8,
    "merge": 9,
    "adamw": 10,
}


class QLoRAError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {_strerror(status)} (status {status})")
        self.status = status


class _Nf4dq(ctypes.Structure):
    _fields_ = [
        ("codes", ctypes.c_void_p),
        ("code8", ctypes.c_void_p),
        ("c2s", ctypes.c_void_p),
        ("mu", ctypes.c_void_p),
        ("d_out", ctypes.c_int64),
        ("d_in", ctypes.c_int64),
        ("block1", ctypes.c_int32),
        ("block2", ctypes.c_int32),
        ("codebook", ctypes.c_int32),
        ("dq_format", ctypes.c_int32),
    ]


_lib = None


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or _LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"HIP library not built: {p} (run python -m bit_nf4_quantized_dq_amd.build)")
    L = ctypes.CDLL(p)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    P = ctypes.POINTER
    sig = {
        "qlora_quant_sizes": (i64, i64, P(sz), P(sz), P(sz)),
        "qlora_workspace_size": (ctypes.c_int, i64, i64, i64, i32, P(sz)),
        "qlora_workspace_size_fmt": (ctypes.c_int, i64, i64, i64, i32, ctypes.c_int, P(sz)),
        "qlora_workspace_init": (vp, sz, vp),
        "qlora_format_sizes": (i64, i64, ctypes.c_int, P(sz), P(sz), P(sz)),
        "qlora_nf4_codebook": (P(ctypes.c_float),),
        "qlora_codebook": (ctypes.c_int, P(ctypes.c_float)),
        "qlora_quantize": (vp, P(_Nf4dq), P(ctypes.c_float), vp, sz, vp),
        "qlora_quantize_bf16": (vp, P(_Nf4dq), P(ctypes.c_float), vp, sz, vp),
        "qlora_dequantize": (P(_Nf4dq), vp, vp),
        "qlora_merge": (P(_Nf4dq), vp, vp, i32, ctypes.c_float, vp, vp),
        "qlora_linear_fwd": (P(_Nf4dq), vp, i64, vp, vp, i32, ctypes.c_float, vp, vp, vp, sz, vp),
        "qlora_linear_fwd_noalloc": (P(_Nf4dq), vp, i64, vp, vp, i32, ctypes.c_float, vp, vp, vp),
        "qlora_linear_bwd": (P(_Nf4dq), vp, vp, i64, vp, vp, i32, ctypes.c_float, vp, vp, vp, vp, vp, sz, vp),
        "qlora_workspace_size_multi": (ctypes.c_int, P(P(_Nf4dq)), i64, i32, P(sz)),
        "qlora_linear_fwd_multi": (ctypes.c_int, P(P(_Nf4dq)), vp, i64, P(vp), P(vp), i32, ctypes.c_float, P(vp),
                                   P(vp), vp, sz, vp),
        "qlora_mlp_workspace_size": (ctypes.c_int, i64, P(_Nf4dq), P(_Nf4dq), P(_Nf4dq), i32, P(sz)),
        "qlora_mlp_fwd": (P(_Nf4dq), P(_Nf4dq), P(_Nf4dq), vp, i64, P(vp), P(vp), i32, ctypes.c_float, vp, vp, vp,
                          vp, sz, vp),
        "qlora_mlp_bwd": (P(_Nf4dq), P(_Nf4dq), P(_Nf4dq), vp, vp, i64, P(vp), P(vp), i32, ctypes.c_float, vp, vp,
                          vp, P(vp), P(vp), vp, sz, vp),
        "qlora_adamw_step": (vp, vp, vp, vp, vp, i64, i64, ctypes.c_float, ctypes.c_float, ctypes.c_float,
                             ctypes.c_float, ctypes.c_float, vp),
        "qlora_e4m3_encode": (vp, vp, i64, vp),
        "qlora_timing_enable": (ctypes.c_int,),
        "qlora_timing_read": (ctypes.c_int, P(ctypes.c_double), P(i64)),
        "qlora_strerror": (ctypes.c_int,),
    }
    for name, args in sig.items():
        fn = getattr(L, name)
        fn.argtypes = list(args)
        fn.restype = ctypes.c_int
    L.qlora_strerror.restype = ctypes.c_char_p
    _lib = L
    return L


class _LazyLib:
    def __getattr__(self, name):
        return getattr(load_library(), name)


lib = _LazyLib()


def _strerror(status: int) -> str:
    try:
        return load_library().qlora_strerror(status).decode()
    except Exception:  # noqa: BLE001
        return "?"


def _check(status: int, what: str) -> None:
    if status != 0:
        raise QLoRAError(status, what)


def _stream(t: torch.Tensor | None = None) -> int:
    dev = t.device if t is not None else torch.device("cuda")
    return torch.cuda.current_stream(dev).cuda_stream


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _dev(t: torch.Tensor, dtype, name: str, shape=None, device=None) -> None:
    """Check one tensor before its pointer crosses the C ABI (see _validate)."""
    _validate([(t, dtype, name, shape)], device)


def _validate(specs, device=None) -> None:
    """Check tensors before their pointers cross the C ABI, which cannot see sizes: each spec
    (tensor, dtype, name, shape or None) must be a contiguous tensor of that dtype and shape;
    then each must be a CUDA tensor on `device` (when given).  All shapes and dtypes are
    checked before any placement, so a wrong size is reported as such wherever it lives."""
    for t, dtype, name, shape in specs:
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{name}: need a torch tensor, got {type(t).__name__}")
        if shape is not None and tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name}: need shape {tuple(shape)}, got {tuple(t.shape)}")
        if t.dtype != dtype or not t.is_contiguous():
            raise ValueError(f"{name}: need a contiguous {dtype} tensor, got {t.dtype}")
    for t, dtype, name, shape in specs:
        if not t.is_cuda:
            raise ValueError(f"{name}: need a CUDA tensor, got one on {t.device}")
        if device is not None and t.device != device:
            raise ValueError(f"{name}: on {t.device}, the other operands are on {device}")


def _weight_specs(q: "QuantizedWeight", prefix: str = "weight"):
    """Specs of the quantized weight's buffers: the sizes its shape and format need."""
    nc, n8, n2 = quant_sizes(q.d_out, q.d_in, q.dq)
    specs = [(q.codes, torch.uint8, f"{prefix}.codes", (nc,)), (q.code8, torch.uint8, f"{prefix}.code8", (n8,))]
    if q.dq != "none":
        specs += [(q.c2s, torch.float32, f"{prefix}.c2s", (n2 // 4,)), (q.mu, torch.float32, f"{prefix}.mu", (1,))]
    return specs


def _check_weight(q: "QuantizedWeight", device=None) -> None:
    _validate(_weight_specs(q), device)


def _check_ws(ws: torch.Tensor, device) -> None:
    if not isinstance(ws, torch.Tensor) or not ws.is_cuda or not ws.is_contiguous() or ws.dtype != torch.uint8:
        raise ValueError("ws: need a contiguous uint8 CUDA tensor")
    if ws.device != device:
        raise ValueError(f"ws: on {ws.device}, the operands are on {device}")


def _rank(A: torch.Tensor, name: str = "A") -> int:
    if not isinstance(A, torch.Tensor) or A.dim() != 2:
        raise ValueError(f"{name}: need a 2-D [r, d_in] tensor")
    return A.shape[0]


def _tokens(X: torch.Tensor, name: str = "X") -> int:
    if not isinstance(X, torch.Tensor) or X.dim() != 2:
        raise ValueError(f"{name}: need a 2-D [M, d] tensor")
    return X.shape[0]


@functools.lru_cache(maxsize=1024)
def quant_sizes(d_out: int, d_in: int, dq: str = "e4m3") -> tuple[int, int, int]:
    a, b, c = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(load_library().qlora_format_sizes(d_out, d_in, DQ_FORMATS[dq], ctypes.byref(a), ctypes.byref(b),
                                             ctypes.byref(c)), "quant_sizes")
    return a.value, b.value, c.value


@functools.lru_cache(maxsize=4096)
def workspace_size(op: int, M: int, d_out: int, d_in: int, r: int, dq: str = "e4m3") -> int:
    n = ctypes.c_size_t()
    _check(load_library().qlora_workspace_size_fmt(op, M, d_out, d_in, r, DQ_FORMATS[dq], ctypes.byref(n)),
           "workspace_size")
    return n.value


def nf4_codebook() -> list[float]:
    arr = (ctypes.c_float * 16)()
    _check(load_library().qlora_nf4_codebook(arr), "nf4_codebook")
    return list(arr)


def codebook(name: str = "nf4") -> list[float]:
    arr = (ctypes.c_float * 16)()
    _check(load_library().qlora_codebook(CODEBOOKS[name], arr), "codebook")
    return list(arr)


@dataclasses.dataclass
class QuantizedWeight:
    """Device buffers of one NF4 + DQ tensor (owned by these torch tensors)."""

    codes: torch.Tensor  # uint8 [d_out * d_in / 2]
    code8: torch.Tensor  # uint8 [d_out * d_in / 64] (uint8 [4 * ...] holding FP32 when dq == "none")
    c2s: torch.Tensor  # float32 [ceil(n_blocks / 256)] (empty when dq == "none")
    mu: torch.Tensor  # float32 [1]
    d_out: int
    d_in: int
    codebook: str = "nf4"
    dq: str = "e4m3"

    @classmethod
    def empty(cls, d_out: int, d_in: int, device="cuda", codebook: str = "nf4", dq: str = "e4m3") -> "QuantizedWeight":
        nc, n8, n2 = quant_sizes(d_out, d_in, dq)
        return cls(
            codes=torch.empty(nc, dtype=torch.uint8, device=device),
            code8=torch.empty(n8, dtype=torch.uint8, device=device),
            c2s=torch.empty(max(n2 // 4, 1), dtype=torch.float32, device=device),
            mu=torch.empty(1, dtype=torch.float32, device=device),
            d_out=d_out,
            d_in=d_in,
            codebook=codebook,
            dq=dq,
        )

    def struct(self) -> _Nf4dq:
        return _Nf4dq(self.codes.data_ptr(), self.code8.data_ptr(), self.c2s.data_ptr(), self.mu.data_ptr(),
                      self.d_out, self.d_in, 64, 256, CODEBOOKS[self.codebook], DQ_FORMATS[self.dq])

    def stored_constants(self) -> torch.Tensor:
        """The per-block constants as stored: E4M3/E5M2/INT8 bytes, or FP32 without DQ."""
        return self.code8.view(torch.float32) if self.dq == "none" else self.code8

    def nbytes(self) -> int:
        extra = 0 if self.dq == "none" else 4 * self.c2s.numel() + 4
        return self.codes.numel() + self.code8.numel() + extra


def new_workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A workspace of `nbytes` bytes ready for its first use: zero-filled, so its counter
    head (the first QLORA_WS_COUNTER_BYTES bytes) starts at zero, as every call leaves it."""
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def workspace_init(ws: torch.Tensor) -> torch.Tensor:
    """Zero the counter head of a workspace that was not allocated zero-filled."""
    if not isinstance(ws, torch.Tensor) or not ws.is_cuda or not ws.is_contiguous() or ws.dtype != torch.uint8:
        raise ValueError("ws: need a contiguous uint8 CUDA tensor")
    _check(load_library().qlora_workspace_init(ws.data_ptr(), ws.numel(), _stream(ws)), "workspace_init")
    return ws


class _Workspace:
    """Scratch buffers grown on demand, one per (device, stream, kind): calls on different
    streams never share one, so they may overlap (calls that share a workspace must not)."""

    def __init__(self):
        self._bufs: dict = {}

    def get(self, nbytes: int, device: torch.device, key: str = "ws") -> torch.Tensor:
        idx = device.index if device.index is not None else torch.cuda.current_device()
        k = (idx, torch.cuda.current_stream(idx).cuda_stream, key)
        buf = self._bufs.get(k)
        if buf is None or buf.numel() < nbytes:
            buf = new_workspace(nbytes, torch.device("cuda", idx))
            self._bufs[k] = buf
        return buf


_WS = _Workspace()


def quantize(W: torch.Tensor, out: QuantizedWeight | None = None, ws: torch.Tensor | None = None,
             codebook: str = "nf4", dq: str = "e4m3") -> QuantizedWeight:
    """Quantize an FP32 [d_out, d_in] CUDA tensor (synchronizes the current stream once).
    The format comes from `out` when given, else from `codebook` and `dq`."""
    return _quantize(W, torch.float32, "qlora_quantize", out, ws, codebook, dq)


def _quantize(W, dtype, fn, out, ws, codebook, dq):
    if not isinstance(W, torch.Tensor) or W.dim() != 2:
        raise ValueError("W: need a 2-D [d_out, d_in] tensor")
    d_out, d_in = W.shape
    if out is not None and (out.d_out, out.d_in) != (d_out, d_in):
        raise ValueError(f"out: a {out.d_out}x{out.d_in} weight cannot hold a {d_out}x{d_in} tensor")
    _dev(W, dtype, "W")
    q = out if out is not None else QuantizedWeight.empty(d_out, d_in, W.device, codebook, dq)
    _check_weight(q, W.device)
    need = workspace_size(OP_QUANTIZE, 1, d_out, d_in, 1)
    ws = ws if ws is not None else _WS.get(need, W.device, "quant")
    _check_ws(ws, W.device)
    mu = ctypes.c_float()
    s = q.struct()
    _check(getattr(load_library(), fn)(W.data_ptr(), ctypes.byref(s), ctypes.byref(mu), ws.data_ptr(), ws.numel(),
                                       _stream(W)), fn[len("qlora_"):])
    return q


def quantize_bf16(W: torch.Tensor, out: QuantizedWeight | None = None, ws: torch.Tensor | None = None,
                  codebook: str = "nf4", dq: str = "e4m3") -> QuantizedWeight:
    """Quantize a BF16 [d_out, d_in] CUDA tensor (its exact FP32 values; synchronizes once)."""
    return _quantize(W, torch.bfloat16, "qlora_quantize_bf16", out, ws, codebook, dq)


def merge(q: QuantizedWeight, A: torch.Tensor, B: torch.Tensor, alpha: float,
          out: torch.Tensor | None = None) -> torch.Tensor:
    """Merged BF16 [d_out, d_in] weight bf16(w_hat + (alpha/r) B A) for export."""
    r = _rank(A)
    dev = A.device
    specs = _weight_specs(q) + [(A, torch.bfloat16, "A", (r, q.d_in)), (B, torch.bfloat16, "B", (q.d_out, r))]
    if out is not None:
        specs.append((out, torch.bfloat16, "out", (q.d_out, q.d_in)))
    _validate(specs, dev)
    out = out if out is not None else torch.empty(q.d_out, q.d_in, dtype=torch.bfloat16, device=dev)
    s = q.struct()
    _check(load_library().qlora_merge(ctypes.byref(s), A.data_ptr(), B.data_ptr(), r, float(alpha), out.data_ptr(),
                                      _stream(out)), "merge")
    return out


def dequantize(q: QuantizedWeight, out: torch.Tensor | None = None) -> torch.Tensor:
    """BF16 [d_out, d_in] w_hat, bit-exact."""
    dev = q.codes.device
    specs = _weight_specs(q)
    if out is not None:
        specs.append((out, torch.bfloat16, "out", (q.d_out, q.d_in)))
    _validate(specs, dev)
    out = out if out is not None else torch.empty(q.d_out, q.d_in, dtype=torch.bfloat16, device=dev)
    s = q.struct()
    _check(load_library().qlora_dequantize(ctypes.byref(s), out.data_ptr(), _stream(out)), "dequantize")
    return out


def linear_fwd(q: QuantizedWeight, X: torch.Tensor, A: torch.Tensor, B: torch.Tensor, alpha: float,
               Y: torch.Tensor | None = None, T_save: torch.Tensor | None = None,
               ws: torch.Tensor | None = None) -> torch.Tensor:
    """Y = X w_hat^T + (alpha/r) (X A^T) B^T.  X [M, d_in], A [r, d_in], B [d_out, r] BF16."""
    M, r, dev = _tokens(X), _rank(A), X.device
    specs = _weight_specs(q) + [(X, torch.bfloat16, "X", (M, q.d_in)), (A, torch.bfloat16, "A", (r, q.d_in)),
                                (B, torch.bfloat16, "B", (q.d_out, r))]
    if Y is not None:
        specs.append((Y, torch.bfloat16, "Y", (M, q.d_out)))
    if T_save is not None:
        specs.append((T_save, torch.bfloat16, "T_save", (M, r)))
    _validate(specs, dev)
    Y = Y if Y is not None else torch.empty(M, q.d_out, dtype=torch.bfloat16, device=dev)
    need = workspace_size(OP_FWD, M, q.d_out, q.d_in, r, q.dq)
    ws = ws if ws is not None else _WS.get(need, dev, "fwd")
    _check_ws(ws, dev)
    s = q.struct()
    _check(load_library().qlora_linear_fwd(ctypes.byref(s), X.data_ptr(), M, A.data_ptr(), B.data_ptr(), r,
                                           float(alpha), Y.data_ptr(), _ptr(T_save), ws.data_ptr(), ws.numel(),
                                           _stream(X)), "linear_fwd")
    return Y


def linear_fwd_noalloc(q: QuantizedWeight, X: torch.Tensor, A: torch.Tensor, B: torch.Tensor, alpha: float,
                       Y: torch.Tensor, T_save: torch.Tensor | None = None) -> torch.Tensor:
    """linear_fwd on the library's fixed per-device scratch: no workspace, and no allocation
    anywhere in the call (Y must be given).  Refused (status -7) when the call needs more than
    QLORA_NOALLOC_SCRATCH_BYTES; calls that overlap on one device race."""
    M, r, dev = _tokens(X), _rank(A), X.device
    specs = _weight_specs(q) + [(X, torch.bfloat16, "X", (M, q.d_in)), (A, torch.bfloat16, "A", (r, q.d_in)),
                                (B, torch.bfloat16, "B", (q.d_out, r)), (Y, torch.bfloat16, "Y", (M, q.d_out))]
    if T_save is not None:
        specs.append((T_save, torch.bfloat16, "T_save", (M, r)))
    _validate(specs, dev)
    s = q.struct()
    _check(load_library().qlora_linear_fwd_noalloc(ctypes.byref(s), X.data_ptr(), M, A.data_ptr(), B.data_ptr(), r,
                                                   float(alpha), Y.data_ptr(), _ptr(T_save), _stream(X)),
           "linear_fwd_noalloc")
    return Y


def _struct_array(qs):
    """Host array of pointers to descriptor structs (the structs are kept alive with it)."""
    structs = [q.struct() for q in qs]
    arr = (ctypes.POINTER(_Nf4dq) * len(qs))(*[ctypes.pointer(x) for x in structs])
    return arr, structs


def workspace_size_multi(qs, M: int, r: int) -> int:
    arr, _keep = _struct_array(qs)
    n = ctypes.c_size_t()
    _check(load_library().qlora_workspace_size_multi(len(qs), arr, M, r, ctypes.byref(n)), "workspace_size_multi")
    return n.value


def linear_fwd_multi(qs, X: torch.Tensor, As, Bs, alpha: float, Ys=None, T_saves=None,
                     ws: torch.Tensor | None = None):
    """Forward of up to 4 linears that read the same X (e.g. q, k, v): returns the list of Y[i]."""
    qs = list(qs)
    n = len(qs)
    if n < 1 or len(As) != n or len(Bs) != n or (Ys is not None and len(Ys) != n) or \
            (T_saves is not None and len(T_saves) != n):
        raise ValueError("linear_fwd_multi: need one A, B (and Y, T_save when given) per weight")
    M, r, dev = _tokens(X), _rank(As[0], "A[0]"), X.device
    specs = [(X, torch.bfloat16, "X", (M, qs[0].d_in))]
    for i, q in enumerate(qs):
        specs += _weight_specs(q, f"weight[{i}]") + [(As[i], torch.bfloat16, f"A[{i}]", (r, q.d_in)),
                                                     (Bs[i], torch.bfloat16, f"B[{i}]", (q.d_out, r))]
        if Ys is not None:
            specs.append((Ys[i], torch.bfloat16, f"Y[{i}]", (M, q.d_out)))
        if T_saves is not None and T_saves[i] is not None:
            specs.append((T_saves[i], torch.bfloat16, f"T_save[{i}]", (M, r)))
    _validate(specs, dev)
    Ys = list(Ys) if Ys is not None else [torch.empty(M, q.d_out, dtype=torch.bfloat16, device=dev) for q in qs]
    need = workspace_size_multi(qs, M, r)
    ws = ws if ws is not None else _WS.get(need, dev, "fwd")
    _check_ws(ws, dev)
    arr, _keep = _struct_array(qs)
    VP = ctypes.c_void_p * n
    a_ptrs, b_ptrs, y_ptrs = VP(*[a.data_ptr() for a in As]), VP(*[b.data_ptr() for b in Bs]), VP(*[y.data_ptr() for y in Ys])
    t_ptrs = None
    if T_saves is not None:
        t_ptrs = VP(*[_ptr(t) for t in T_saves])
    _check(load_library().qlora_linear_fwd_multi(n, arr, X.data_ptr(), M, a_ptrs, b_ptrs, r, float(alpha), y_ptrs,
                                                 t_ptrs, ws.data_ptr(), ws.numel(), _stream(X)), "linear_fwd_multi")
    return Ys


def mlp_workspace_size(op: int, M: int, qg: QuantizedWeight, qu: QuantizedWeight, qd: QuantizedWeight,
                       r: int) -> int:
    n = ctypes.c_size_t()
    sg, su, sd = qg.struct(), qu.struct(), qd.struct()
    _check(load_library().qlora_mlp_workspace_size(op, M, ctypes.byref(sg), ctypes.byref(su), ctypes.byref(sd), r,
                                                   ctypes.byref(n)), "mlp_workspace_size")
    return n.value


def _ptrs(ts):
    return (ctypes.c_void_p * len(ts))(*[t.data_ptr() for t in ts])


def _mlp_specs(qs, As, Bs, r):
    if len(qs) != 3 or len(As) != 3 or len(Bs) != 3:
        raise ValueError("MLP block: need the three weights and adapters gate, up, down")
    specs = []
    for i, q in enumerate(qs):
        specs += _weight_specs(q, f"weight[{i}]") + [(As[i], torch.bfloat16, f"A[{i}]", (r, q.d_in)),
                                                     (Bs[i], torch.bfloat16, f"B[{i}]", (q.d_out, r))]
    return specs


def mlp_fwd(qs, X: torch.Tensor, As, Bs, alpha: float, Y: torch.Tensor | None = None,
            G_save: torch.Tensor | None = None, U_save: torch.Tensor | None = None,
            ws: torch.Tensor | None = None) -> torch.Tensor:
    """MLP block Y = down(silu(gate(X)) * up(X)); qs, As, Bs in the order gate, up, down."""
    qg, qu, qd = qs
    M, r, dev = _tokens(X), _rank(As[0], "A[0]"), X.device
    d, f = qg.d_in, qg.d_out
    specs = _mlp_specs(qs, As, Bs, r) + [(X, torch.bfloat16, "X", (M, d))]
    if Y is not None:
        specs.append((Y, torch.bfloat16, "Y", (M, qd.d_out)))
    for t, n in ((G_save, "G_save"), (U_save, "U_save")):
        if t is not None:
            specs.append((t, torch.bfloat16, n, (M, f)))
    _validate(specs, dev)
    Y = Y if Y is not None else torch.empty(M, qd.d_out, dtype=torch.bfloat16, device=dev)
    need = mlp_workspace_size(OP_FWD, M, qg, qu, qd, r)
    ws = ws if ws is not None else _WS.get(need, dev, "fwd")
    _check_ws(ws, dev)
    sg, su, sd = qg.struct(), qu.struct(), qd.struct()
    _check(load_library().qlora_mlp_fwd(ctypes.byref(sg), ctypes.byref(su), ctypes.byref(sd), X.data_ptr(), M,
                                        _ptrs(As), _ptrs(Bs), r, float(alpha), Y.data_ptr(), _ptr(G_save),
                                        _ptr(U_save), ws.data_ptr(), ws.numel(), _stream(X)), "mlp_fwd")
    return Y


def mlp_bwd(qs, X: torch.Tensor, dY: torch.Tensor, As, Bs, alpha: float, G_saved: torch.Tensor | None = None,
            U_saved: torch.Tensor | None = None, dX: torch.Tensor | None = None, ws: torch.Tensor | None = None):
    """Backward of mlp_fwd: returns (dX, [dA_gate, dA_up, dA_down], [dB_gate, dB_up, dB_down])."""
    qg, qu, qd = qs
    M, r, dev = _tokens(X), _rank(As[0], "A[0]"), X.device
    d, f = qg.d_in, qg.d_out
    if (G_saved is None) != (U_saved is None):
        raise ValueError("mlp_bwd: give both G_saved and U_saved, or neither")
    specs = _mlp_specs(qs, As, Bs, r) + [(X, torch.bfloat16, "X", (M, d)), (dY, torch.bfloat16, "dY", (M, qd.d_out))]
    for t, n in ((G_saved, "G_saved"), (U_saved, "U_saved"), (dX, "dX")):
        if t is not None:
            specs.append((t, torch.bfloat16, n, (M, d if n == "dX" else f)))
    _validate(specs, dev)
    dX = dX if dX is not None else torch.empty(M, d, dtype=torch.bfloat16, device=dev)
    dAs = [torch.empty(r, q.d_in, dtype=torch.bfloat16, device=dev) for q in qs]
    dBs = [torch.empty(q.d_out, r, dtype=torch.bfloat16, device=dev) for q in qs]
    need = mlp_workspace_size(OP_BWD, M, qg, qu, qd, r)
    ws = ws if ws is not None else _WS.get(need, dev, "bwd")
    _check_ws(ws, dev)
    sg, su, sd = qg.struct(), qu.struct(), qd.struct()
    _check(load_library().qlora_mlp_bwd(ctypes.byref(sg), ctypes.byref(su), ctypes.byref(sd), X.data_ptr(),
                                        dY.data_ptr(), M, _ptrs(As), _ptrs(Bs), r, float(alpha), _ptr(G_saved),
                                        _ptr(U_saved), dX.data_ptr(), _ptrs(dAs), _ptrs(dBs), ws.data_ptr(),
                                        ws.numel(), _stream(X)), "mlp_bwd")
    return dX, dAs, dBs


def linear_bwd(q: QuantizedWeight, X: torch.Tensor, dY: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
               alpha: float, T_saved: torch.Tensor | None = None, need_dX: bool = True,
               dX: torch.Tensor | None = None, dA: torch.Tensor | None = None, dB: torch.Tensor | None = None,
               ws: torch.Tensor | None = None):
    """Returns (dX or None, dA, dB), all BF16."""
    M, r, dev = _tokens(X), _rank(A), X.device
    specs = _weight_specs(q) + [(X, torch.bfloat16, "X", (M, q.d_in)), (dY, torch.bfloat16, "dY", (M, q.d_out)),
                                (A, torch.bfloat16, "A", (r, q.d_in)), (B, torch.bfloat16, "B", (q.d_out, r))]
    for t, n, shp in ((T_saved, "T_saved", (M, r)), (dX if need_dX else None, "dX", (M, q.d_in)),
                      (dA, "dA", (r, q.d_in)), (dB, "dB", (q.d_out, r))):
        if t is not None:
            specs.append((t, torch.bfloat16, n, shp))
    _validate(specs, dev)
    if need_dX and dX is None:
        dX = torch.empty(M, q.d_in, dtype=torch.bfloat16, device=dev)
    dA = dA if dA is not None else torch.empty(r, q.d_in, dtype=torch.bfloat16, device=dev)
    dB = dB if dB is not None else torch.empty(q.d_out, r, dtype=torch.bfloat16, device=dev)
    need = workspace_size(OP_BWD, M, q.d_out, q.d_in, r, q.dq)
    ws = ws if ws is not None else _WS.get(need, dev, "bwd")
    _check_ws(ws, dev)
    s = q.struct()
    _check(load_library().qlora_linear_bwd(ctypes.byref(s), X.data_ptr(), dY.data_ptr(), M, A.data_ptr(),
                                           B.data_ptr(), r, float(alpha), _ptr(T_saved),
                                           _ptr(dX if need_dX else None), dA.data_ptr(), dB.data_ptr(),
                                           ws.data_ptr(), ws.numel(), _stream(X)), "linear_bwd")
    return (dX if need_dX else None), dA, dB


def adamw_step(master: torch.Tensor, m: torch.Tensor, v: torch.Tensor, grad: torch.Tensor, step: int, lr: float,
               beta1: float = 0.9, beta2: float = 0.999, eps: float = 1e-8, weight_decay: float = 0.0,
               param: torch.Tensor | None = None) -> None:
    """One AdamW step, in place, over flat FP32 master/m/v with a BF16 gradient; writes the
    BF16 working copy into `param` when given."""
    for t, n in ((master, "master"), (m, "m"), (v, "v")):
        _dev(t, torch.float32, n)
    _dev(grad, torch.bfloat16, "grad")
    if param is not None:
        _dev(param, torch.bfloat16, "param")
    n = master.numel()
    if any(t.numel() != n for t in (m, v, grad)) or (param is not None and param.numel() != n):
        raise ValueError("adamw_step: all buffers need the same number of elements")
    _check(load_library().qlora_adamw_step(master.data_ptr(), m.data_ptr(), v.data_ptr(), grad.data_ptr(),
                                           _ptr(param), n, int(step), float(lr), float(beta1), float(beta2),
                                           float(eps), float(weight_decay), _stream(master)), "adamw_step")


def e4m3_encode(x: torch.Tensor) -> torch.Tensor:
    _dev(x, torch.float32, "x")
    out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _check(load_library().qlora_e4m3_encode(x.data_ptr(), out.data_ptr(), x.numel(), _stream(x)), "e4m3_encode")
    return out


def timing_enable(on, kernels=None) -> None:
    """Per-launch HIP events for the named kernels (all of them when `kernels` is None);
    on=False turns timing off."""
    if not on:
        mask = 0
    elif kernels is None:
        mask = (1 << len(KERNEL_IDS)) - 1
    else:
        mask = 0
        for k in kernels:
            mask |= 1 << KERNEL_IDS[k]
    _check(load_library().qlora_timing_enable(mask), "timing_enable")


def timing_read(kernel: str) -> tuple[float, int]:
    """(total ms, launches) of one kernel since the last read; waits for its events."""
    ms, n = ctypes.c_double(), ctypes.c_int64()
    _check(load_library().qlora_timing_read(KERNEL_IDS[kernel], ctypes.byref(ms), ctypes.byref(n)), "timing_read")
    return ms.value, n.value
