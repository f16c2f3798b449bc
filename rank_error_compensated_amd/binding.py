"""ctypes binding of libserq.so (include/serq.h), with the same entry-point names.

Argument marshalling only: every step of the layer runs in the library.  Host
entry points take numpy arrays; device entry points take torch tensors, used
only as device memory (``data_ptr()``) and for the current HIP stream.  The
binding raises ``SerqError`` for every non-zero status and refuses to run when
the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int, c_int32, c_int64, c_size_t, c_void_p

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_lib", "libserq.so")

FMT = {"int4": 0, "w4a8": 1, "mxfp4": 2, "mxw4a8": 3}
DTYPE = {"f32": 0, "bf16": 1}

SERQ_OK = 0
SERQ_ERR_INVALID_ARG = -1
SERQ_ERR_SHAPE = -2
SERQ_ERR_UNSUPPORTED = -3
SERQ_ERR_BUFFER = -4
SERQ_ERR_HIP = -5

EXPORTS = ("serq_query_layout", "serq_prepare_weights", "serq_flatten_act", "serq_act_bytes",
           "serq_quant_act", "serq_rmsnorm_quant", "serq_swiglu_quant", "serq_linear_workspace_bytes",
           "serq_linear", "serq_linear_noalloc", "serq_linear_swiglu", "serq_linear_swiglu_q", "serq_linear_q", "serq_status_string", "serq_last_error",
           "serq_prepare_weights_gptq", "serq_weight_error", "serq_l2qer_sizes", "serq_l2qer_prepare", "serq_l2qer_workspace_bytes",
           "serq_l2qer_intermediate", "serq_l2qer_linear_q", "serq_l2qer_linear")


class serq_layout(ctypes.Structure):
    _fields_ = [("d_in", c_int32), ("d_out", c_int32), ("r", c_int32), ("r_pad", c_int32),
                ("fmt", c_int32), ("layout_version", c_int32),
                ("perm_bytes", c_size_t), ("s_bytes", c_size_t), ("wq_bytes", c_size_t),
                ("wscale_bytes", c_size_t), ("rq_bytes", c_size_t), ("rscale_bytes", c_size_t)]

    @property
    def fmt_name(self) -> str:
        return {v: k for k, v in FMT.items()}[self.fmt]


class SerqError(RuntimeError):
    def __init__(self, status: int, text: str, detail: str):
        super().__init__(f"serq status {status} ({text}): {detail}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libserq.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m rank_error_compensated_amd._build`")
    L = ctypes.CDLL(LIB_PATH)
    LP = POINTER(serq_layout)
    sig = {
        "serq_query_layout": (c_int, [c_int32, c_int32, c_int32, c_int, LP]),
        "serq_prepare_weights": (c_int, [LP, c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_void_p,
                                         c_void_p, c_void_p, c_void_p, c_void_p]),
        "serq_flatten_act": (c_int, [c_void_p, c_int64, c_int32, c_void_p, c_void_p, c_void_p]),
        "serq_act_bytes": (c_int, [c_int32, c_int32, c_int, POINTER(c_size_t), POINTER(c_size_t)]),
        "serq_quant_act": (c_int, [c_void_p, c_int, c_int32, c_int32, c_int, c_void_p, c_void_p, c_void_p]),
        "serq_rmsnorm_quant": (c_int, [c_void_p, c_int, c_int32, c_int32, c_void_p, c_float, c_void_p, c_void_p,
                                       c_int, c_void_p, c_void_p, c_void_p]),
        "serq_swiglu_quant": (c_int, [c_void_p, c_int, c_int32, c_int32, c_void_p, c_void_p, c_int, c_void_p,
                                      c_void_p, c_void_p]),
        "serq_linear_workspace_bytes": (c_size_t, [LP, c_int32]),
        "serq_linear": (c_int, [LP, c_void_p, c_int, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                                c_void_p, c_void_p, c_size_t, c_void_p]),
        "serq_linear_noalloc": (c_int, [LP, c_void_p, c_int, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                                        c_void_p, c_void_p]),
        "serq_linear_swiglu": (c_int, [LP, c_void_p, c_int, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                                       c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
        "serq_linear_swiglu_q": (c_int, [LP, c_void_p, c_int, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                                         c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
        "serq_linear_q": (c_int, [LP, c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                                  c_void_p, c_void_p, c_void_p, c_void_p]),
        "serq_prepare_weights_gptq": (c_int, [LP, c_void_p, c_void_p, c_int32, c_float, c_void_p, c_void_p,
                                              c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
        "serq_weight_error": (c_int, [LP, c_void_p, c_void_p, c_int32, c_void_p]),
        "serq_l2qer_sizes": (c_int, [LP, c_int32, POINTER(c_size_t)]),
        "serq_l2qer_prepare": (c_int, [LP, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
        "serq_l2qer_workspace_bytes": (c_size_t, [LP, c_int32, c_int32]),
        "serq_l2qer_intermediate": (c_int, [LP, c_int32, c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_void_p,
                                            c_void_p, c_void_p, c_void_p]),
        "serq_l2qer_linear_q": (c_int, [LP, c_int32, c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_void_p,
                                        c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
        "serq_l2qer_linear": (c_int, [LP, c_int32, c_void_p, c_int, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                                      c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
        "serq_status_string": (c_char_p, [c_int]),
        "serq_last_error": (c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype, fn.argtypes = res, args
    _lib = L
    return L


def _check(st: int) -> None:
    if st != SERQ_OK:
        L = lib()
        raise SerqError(st, L.serq_status_string(st).decode(), L.serq_last_error().decode())


def _fmt(fmt) -> int:
    return FMT[fmt] if isinstance(fmt, str) else int(fmt)


def _ptr(a) -> int | None:
    """Address of a numpy array or torch tensor (None for None)."""
    if a is None:
        return None
    if isinstance(a, np.ndarray):
        assert a.flags["C_CONTIGUOUS"]
        return a.ctypes.data
    assert a.is_contiguous()
    return a.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


# ----------------------------------------------------------------- host calls

def serq_query_layout(d_in: int, d_out: int, r: int, fmt) -> serq_layout:
    out = serq_layout()
    _check(lib().serq_query_layout(d_in, d_out, r, _fmt(fmt), ctypes.byref(out)))
    return out


def serq_prepare_weights(L: serq_layout, W: np.ndarray, X_cal: np.ndarray, want_R: bool = False,
                         gptq_damp: float | None = None) -> dict:
    """Offline preparation on the host; returns the buffers as numpy arrays.
    With gptq_damp set, the non-salient rows are quantized by GPTQ
    (serq_prepare_weights_gptq) instead of round to nearest."""
    W = np.ascontiguousarray(W, np.float32)
    X_cal = np.ascontiguousarray(X_cal, np.float32)
    assert W.shape == (L.d_in, L.d_out) and X_cal.ndim == 2 and X_cal.shape[1] == L.d_in
    out = {
        "perm": np.empty(L.d_in, np.int32),
        "s": np.empty(L.d_in, np.float32),
        "wq": np.empty(L.wq_bytes, np.uint8),              # raw bytes, layout per include/serq.h
        "wscale": np.empty(L.wscale_bytes, np.uint8),
        "rq": np.empty(L.rq_bytes, np.uint8),
        "rscale": np.empty(L.rscale_bytes, np.uint8),
    }
    R = np.empty((L.r, L.d_out), np.float32) if want_R else None
    bufs = (_ptr(out["perm"]), _ptr(out["s"]), _ptr(out["wq"]), _ptr(out["wscale"]), _ptr(out["rq"]),
            _ptr(out["rscale"]), _ptr(R))
    if gptq_damp is None:
        _check(lib().serq_prepare_weights(ctypes.byref(L), _ptr(W), _ptr(X_cal), X_cal.shape[0], *bufs))
    else:
        _check(lib().serq_prepare_weights_gptq(ctypes.byref(L), _ptr(W), _ptr(X_cal), X_cal.shape[0],
                                               float(gptq_damp), *bufs))
    if want_R:
        out["R"] = R
    return out


def serq_flatten_act(X: np.ndarray, perm: np.ndarray, s: np.ndarray) -> np.ndarray:
    X = np.ascontiguousarray(X, np.float32)
    perm = np.ascontiguousarray(perm, np.int32)
    s = np.ascontiguousarray(s, np.float32)
    out = np.empty_like(X)
    _check(lib().serq_flatten_act(_ptr(X), X.shape[0], X.shape[1], _ptr(perm), _ptr(s), _ptr(out)))
    return out


def serq_act_bytes(M: int, d_in: int, fmt) -> tuple:
    a, b = c_size_t(), c_size_t()
    _check(lib().serq_act_bytes(M, d_in, _fmt(fmt), ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def serq_linear_workspace_bytes(L: serq_layout, M: int) -> int:
    return int(lib().serq_linear_workspace_bytes(ctypes.byref(L), M))


# ----------------------------------------------------------------- device calls

def serq_quant_act(X, fmt, xq, xscale, stream=None, M: int | None = None) -> None:
    """X: device tensor [M][d_in] (float32 or bfloat16)."""
    import torch
    xdt = DTYPE["bf16"] if X.dtype == torch.bfloat16 else DTYPE["f32"]
    M = X.shape[0] if M is None else M
    _check(lib().serq_quant_act(_ptr(X), xdt, M, X.shape[1], _fmt(fmt), _ptr(xq), _ptr(xscale),
                                _stream(stream)))


def serq_rmsnorm_quant(H, gamma_p, eps: float, perm, s_p, fmt, xq, xscale, stream=None) -> None:
    """H: device tensor [M][d] (float32 or bfloat16); perm: int32 [d]; gamma_p,
    s_p: float32 [d] in saliency order (gamma[perm], s[perm])."""
    import torch
    xdt = DTYPE["bf16"] if H.dtype == torch.bfloat16 else DTYPE["f32"]
    _check(lib().serq_rmsnorm_quant(_ptr(H), xdt, H.shape[0], H.shape[1], _ptr(gamma_p), float(eps), _ptr(perm),
                                    _ptr(s_p), _fmt(fmt), _ptr(xq), _ptr(xscale), _stream(stream)))


def serq_swiglu_quant(GU, perm, s_p, fmt, xq, xscale, stream=None) -> None:
    """GU: device tensor [M][2 d] (gate half, then up half); perm: int32 [d],
    or None when GU already comes in saliency order; s_p: float32 [d] in
    saliency order (s[perm])."""
    import torch
    xdt = DTYPE["bf16"] if GU.dtype == torch.bfloat16 else DTYPE["f32"]
    assert GU.shape[1] % 2 == 0
    _check(lib().serq_swiglu_quant(_ptr(GU), xdt, GU.shape[0], GU.shape[1] // 2, _ptr(perm), _ptr(s_p), _fmt(fmt),
                                   _ptr(xq), _ptr(xscale), _stream(stream)))


def serq_linear(L: serq_layout, X, wq, wscale, rq, rscale, Y, workspace, stream=None,
                M: int | None = None) -> None:
    import torch
    xdt = DTYPE["bf16"] if X.dtype == torch.bfloat16 else DTYPE["f32"]
    M = X.shape[0] if M is None else M
    _check(lib().serq_linear(ctypes.byref(L), _ptr(X), xdt, M, _ptr(wq), _ptr(wscale), _ptr(rq),
                             _ptr(rscale), _ptr(Y), _ptr(workspace), workspace.numel() * workspace.element_size(),
                             _stream(stream)))


# bytes of device scratch serq_linear_noalloc holds per device (SERQ_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 64 << 20


def serq_linear_noalloc(L: serq_layout, X, wq, wscale, rq, rscale, Y, stream=None, M: int | None = None) -> None:
    import torch
    xdt = DTYPE["bf16"] if X.dtype == torch.bfloat16 else DTYPE["f32"]
    M = X.shape[0] if M is None else M
    _check(lib().serq_linear_noalloc(ctypes.byref(L), _ptr(X), xdt, M, _ptr(wq), _ptr(wscale), _ptr(rq),
                                     _ptr(rscale), _ptr(Y), _stream(stream)))


def serq_linear_swiglu(L: serq_layout, X, wq, wscale, rq, rscale, s_next, H, workspace, stream=None,
                       M: int | None = None) -> None:
    import torch
    xdt = DTYPE["bf16"] if X.dtype == torch.bfloat16 else DTYPE["f32"]
    M = X.shape[0] if M is None else M
    _check(lib().serq_linear_swiglu(ctypes.byref(L), _ptr(X), xdt, M, _ptr(wq), _ptr(wscale), _ptr(rq),
                                    _ptr(rscale), _ptr(s_next), _ptr(H), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), _stream(stream)))


def serq_linear_swiglu_q(L: serq_layout, X, wq, wscale, rq, rscale, s_next, xq_next, xscale_next, workspace,
                         stream=None, M: int | None = None) -> None:
    import torch
    xdt = DTYPE["bf16"] if X.dtype == torch.bfloat16 else DTYPE["f32"]
    M = X.shape[0] if M is None else M
    _check(lib().serq_linear_swiglu_q(ctypes.byref(L), _ptr(X), xdt, M, _ptr(wq), _ptr(wscale), _ptr(rq),
                                      _ptr(rscale), _ptr(s_next), _ptr(xq_next), _ptr(xscale_next), _ptr(workspace),
                                      workspace.numel() * workspace.element_size(), _stream(stream)))


def serq_linear_q(L: serq_layout, xq, xscale, M: int, wq, wscale, rq, rscale, Y, acc_main=None,
                  acc_res=None, stream=None) -> None:
    _check(lib().serq_linear_q(ctypes.byref(L), _ptr(xq), _ptr(xscale), M, _ptr(wq), _ptr(wscale),
                               _ptr(rq), _ptr(rscale), _ptr(Y), _ptr(acc_main), _ptr(acc_res),
                               _stream(stream)))


# ----------------------------------------------------------------- L2QER comparator

def serq_weight_error(L: serq_layout, W: np.ndarray, X_cal: np.ndarray) -> np.ndarray:
    W = np.ascontiguousarray(W, np.float32)
    X_cal = np.ascontiguousarray(X_cal, np.float32)
    E = np.empty((L.d_in, L.d_out), np.float32)
    _check(lib().serq_weight_error(ctypes.byref(L), _ptr(W), _ptr(X_cal), X_cal.shape[0], _ptr(E)))
    return E


def serq_l2qer_sizes(L: serq_layout, k: int) -> tuple:
    sizes = (c_size_t * 4)()
    _check(lib().serq_l2qer_sizes(ctypes.byref(L), k, sizes))
    return tuple(int(v) for v in sizes)


def serq_l2qer_prepare(L: serq_layout, L1: np.ndarray, L2: np.ndarray) -> dict:
    k = L1.shape[1]
    L1 = np.ascontiguousarray(L1, np.float32)
    L2 = np.ascontiguousarray(L2, np.float32)
    n = serq_l2qer_sizes(L, k)
    out = {name: np.zeros(b, np.uint8) for name, b in zip(("l1q", "l1scale", "l2q", "l2scale"), n)}
    _check(lib().serq_l2qer_prepare(ctypes.byref(L), k, _ptr(L1), _ptr(L2), _ptr(out["l1q"]), _ptr(out["l1scale"]),
                                    _ptr(out["l2q"]), _ptr(out["l2scale"])))
    out["k"] = k
    return out


def serq_l2qer_workspace_bytes(L: serq_layout, M: int, k: int) -> int:
    return int(lib().serq_l2qer_workspace_bytes(ctypes.byref(L), M, k))


def serq_l2qer_intermediate(L: serq_layout, k: int, xq, xscale, M: int, l1q, l1scale, T, tq, tscale,
                            stream=None) -> None:
    _check(lib().serq_l2qer_intermediate(ctypes.byref(L), k, _ptr(xq), _ptr(xscale), M, _ptr(l1q), _ptr(l1scale),
                                         _ptr(T), _ptr(tq), _ptr(tscale), _stream(stream)))


def serq_l2qer_linear_q(L: serq_layout, k: int, xq, xscale, M: int, wq, wscale, tq, tscale, l2q, l2scale, Y,
                        stream=None) -> None:
    _check(lib().serq_l2qer_linear_q(ctypes.byref(L), k, _ptr(xq), _ptr(xscale), M, _ptr(wq), _ptr(wscale),
                                     _ptr(tq), _ptr(tscale), _ptr(l2q), _ptr(l2scale), _ptr(Y), _stream(stream)))


def serq_l2qer_linear(L: serq_layout, k: int, X, wq, wscale, l1q, l1scale, l2q, l2scale, Y, workspace,
                      stream=None, M: int | None = None) -> None:
    import torch
    xdt = DTYPE["bf16"] if X.dtype == torch.bfloat16 else DTYPE["f32"]
    M = X.shape[0] if M is None else M
    _check(lib().serq_l2qer_linear(ctypes.byref(L), k, _ptr(X), xdt, M, _ptr(wq), _ptr(wscale), _ptr(l1q),
                                   _ptr(l1scale), _ptr(l2q), _ptr(l2scale), _ptr(Y), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(stream)))


# ----------------------------------------------------------------- convenience

class PreparedLayer:
    """A prepared layer resident in device memory (torch tensors as storage)."""

    def __init__(self, L: serq_layout, host: dict, device: str = "cuda"):
        import torch
        self.L = L
        self.host = host
        self.dev = {k: torch.from_numpy(np.ascontiguousarray(host[k])).to(device)
                    for k in ("wq", "wscale", "rq", "rscale")}

    @classmethod
    def prepare(cls, W: np.ndarray, X_cal: np.ndarray, r: int, fmt, device: str = "cuda",
                gptq_damp: float | None = None):
        L = serq_query_layout(W.shape[0], W.shape[1], r, fmt)
        return cls(L, serq_prepare_weights(L, W, X_cal, gptq_damp=gptq_damp), device)

    def workspace(self, M: int):
        import torch
        return torch.empty(serq_linear_workspace_bytes(self.L, M), dtype=torch.uint8,
                           device=self.dev["wq"].device)

    def __call__(self, X, Y=None, workspace=None, stream=None):
        import torch
        M = X.shape[0]
        if Y is None:
            Y = torch.empty((M, self.L.d_out), dtype=torch.float32, device=X.device)
        if workspace is None:
            workspace = self.workspace(M)
        d = self.dev
        serq_linear(self.L, X, d["wq"], d["wscale"], d["rq"], d["rscale"], Y, workspace, stream)
        return Y
