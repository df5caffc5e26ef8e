"""Python binding of libpsffn, the predictor-gated neuron-level sparse FFN for MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP kernels of
``libpsffn.so`` behind the C ABI in ``include/psffn.h``.  torch is used for device memory and the
current stream.  There is no CPU fallback: importing this package without the built library
raises.

Calls mirror the C ABI by name:
    workspace_bytes, workspace_init, predict, compact, sparse_ffn, profile_counts,
    permute_hot_first, layernorm_f16, status_str
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass, replace
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# PSFFN_LIB names another build of the same library (the host-sanitizer test loads one whose host code
# is built with ASan + UBSan); there is no fallback when the library is missing
LIB_PATH = os.environ.get("PSFFN_LIB") or os.path.join(_HERE, "libpsffn.so")

PSFFN_OK, PSFFN_E_INVALID_ARG, PSFFN_E_UNSUPPORTED, PSFFN_E_WORKSPACE, PSFFN_E_HIP = range(5)
PSFFN_F32, PSFFN_F16, PSFFN_I4G128 = 0, 1, 2
PSFFN_RELU, PSFFN_SWIGLU = 0, 1
MAX_BATCH = 32

if not os.path.exists(LIB_PATH):
    raise ImportError("libpsffn.so is not built (run: python activation_sparse_ffn_psffn_amd/build.py); "
                      "there is no fallback implementation")
_lib = ctypes.CDLL(LIB_PATH)

_vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t


class _Predictor(ctypes.Structure):
    _fields_ = [("d", _i), ("F", _i), ("r", _i), ("dt", _i), ("A", _vp), ("Q", _vp), ("c", _vp)]


class _FFN(ctypes.Structure):
    _fields_ = [("d", _i), ("F", _i), ("dt", _i), ("act", _i), ("w_up", _vp), ("w_gate", _vp), ("w_dT", _vp),
                ("s_up", _vp), ("s_gate", _vp), ("s_dT", _vp), ("b_up", _vp), ("b_gate", _vp), ("b_down", _vp)]


_P = ctypes.POINTER
_lib.psffn_status_str.restype = ctypes.c_char_p
_lib.psffn_status_str.argtypes = [_i]
_lib.psffn_workspace_bytes.restype = _sz
_lib.psffn_workspace_bytes.argtypes = [_P(_Predictor), _P(_FFN), _i]
_lib.psffn_workspace_init.restype = _i
_lib.psffn_workspace_init.argtypes = [_vp, _sz, _vp]
_lib.psffn_predict.restype = _i
_lib.psffn_predict.argtypes = [_P(_Predictor), _vp, _i, _f, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.psffn_compact.restype = _i
_lib.psffn_compact.argtypes = [_vp, _i, _i, _f, _vp, _vp, _vp, _sz, _vp]
_lib.psffn_sparse_ffn.restype = _i
_lib.psffn_sparse_ffn.argtypes = [_P(_FFN), _vp, _i, _vp, _vp, _vp, _i, _vp, _sz, _vp]
_lib.psffn_layer.restype = _i
_lib.psffn_layer.argtypes = [_P(_Predictor), _P(_FFN), _vp, _i, _f, _vp, _vp, _vp, _vp, _i, _vp, _sz, _vp]
_lib.psffn_predict_hot.restype = _i
_lib.psffn_predict_hot.argtypes = [_P(_Predictor), _i, _vp, _i, _f, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.psffn_layer_hot.restype = _i
_lib.psffn_layer_hot.argtypes = [_P(_Predictor), _P(_FFN), _i, _vp, _i, _f, _vp, _vp, _vp, _vp, _i, _vp, _sz, _vp]
_lib.psffn_layer_ln.restype = _i
_lib.psffn_layer_ln.argtypes = [_P(_Predictor), _P(_FFN), _vp, _f, _vp, _i, _f, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.psffn_layer_noalloc.restype = _i
_lib.psffn_layer_noalloc.argtypes = [_P(_Predictor), _P(_FFN), _vp, _i, _f, _vp, _vp, _vp, _vp, _i, _vp]
_lib.psffn_profile_counts.restype = _i
_lib.psffn_profile_counts.argtypes = [_P(_FFN), _vp, _i, _vp, _vp]
_lib.psffn_permute_hot_first.restype = _i
_lib.psffn_permute_hot_first.argtypes = [_vp, _i, _vp, _P(_FFN), _P(_FFN), _P(_Predictor), _P(_Predictor), _vp]
_lib.psffn_layernorm_f16.restype = _i
_lib.psffn_layernorm_f16.argtypes = [_vp, _i, _i, _f, _vp, _vp]

EXPORTED = ("psffn_status_str", "psffn_workspace_bytes", "psffn_workspace_init", "psffn_predict", "psffn_compact",
            "psffn_sparse_ffn", "psffn_layer", "psffn_predict_hot", "psffn_layer_hot", "psffn_layer_ln",
            "psffn_layer_noalloc",
            "psffn_profile_counts",
            "psffn_permute_hot_first",
            "psffn_layernorm_f16")


class PsffnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (status %d)" % (where, status_str(status), status))


def status_str(status: int) -> str:
    return _lib.psffn_status_str(int(status)).decode()


def _check(status: int, where: str):
    if status != PSFFN_OK:
        raise PsffnError(status, where)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dt(t: torch.Tensor) -> int:
    dt = {torch.float32: PSFFN_F32, torch.float16: PSFFN_F16, torch.uint8: PSFFN_I4G128}.get(t.dtype)
    if dt is None:
        raise ValueError("weights must be float32, float16 or uint8 (packed 4-bit), got %s" % t.dtype)
    return dt


# ---- argument checks: the C ABI sees raw pointers only, so shapes, dtypes, contiguity and devices
# are checked here before any call (ValueError), as a wrong one would read or write outside a buffer.

def _req(t, name: str, dtype=None, shape=None, min_numel=None, device=None, gpu=True) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise ValueError("%s: expected a tensor, got %s" % (name, type(t).__name__))
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s: expected dtype %s, got %s" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s: expected shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError("%s: needs at least %d elements, has %d" % (name, min_numel, t.numel()))
    if not t.is_contiguous():
        raise ValueError("%s: must be contiguous" % name)
    if device is not None and t.device != device:
        raise ValueError("%s: on %s, expected %s" % (name, t.device, device))
    if gpu and t.device.type != "cuda":
        raise ValueError("%s: must be a GPU tensor (the library takes device pointers), got %s" % (name, t.device))
    return t


def _act_dtype(storage_dtype) -> torch.dtype:
    # activations are fp32 for fp32 weights, else fp16
    return torch.float32 if storage_dtype == torch.float32 else torch.float16


def _batch(x: torch.Tensor, d: int, dtype, name="x") -> int:
    if x.dim() != 2:
        raise ValueError("%s: expected [B][d], got shape %s" % (name, tuple(x.shape)))
    B = x.shape[0]
    if not 1 <= B <= MAX_BATCH:
        raise ValueError("%s: batch %d outside 1..%d" % (name, B, MAX_BATCH))
    _req(x, name, dtype=dtype, shape=(B, d))
    return B


def _outs(dev, F: int, idx, count, logits=None, B=None, y=None, d=None, ws=None):
    if idx is not None:
        _req(idx, "idx", dtype=torch.int32, min_numel=F, device=dev)
    if count is not None:
        _req(count, "count", dtype=torch.int32, min_numel=1, device=dev)
    if logits is not None:
        _req(logits, "logits", dtype=torch.float32, shape=(B, F), device=dev)
    if y is not None:
        _req(y, "y", dtype=torch.float32, shape=(B, d), device=dev)
    if ws is not None:
        _req(ws, "ws", dtype=torch.uint8, device=dev)


@dataclass
class Predictor:
    """Low-rank predictor of one layer: A [r][d], Q [F][r] (fp32 or fp16, same type), c [F] fp32."""
    A: torch.Tensor
    Q: torch.Tensor
    c: torch.Tensor

    def check(self) -> "Predictor":
        if self.A.dim() != 2 or self.Q.dim() != 2:
            raise ValueError("Predictor: A must be [r][d] and Q [F][r]")
        r, d = self.A.shape
        F = self.Q.shape[0]
        if self.A.dtype not in (torch.float32, torch.float16):
            raise ValueError("Predictor: A must be float32 or float16, got %s" % self.A.dtype)
        dev = self.A.device
        _req(self.A, "Predictor.A", device=dev, gpu=False)
        _req(self.Q, "Predictor.Q", dtype=self.A.dtype, shape=(F, r), device=dev, gpu=False)
        _req(self.c, "Predictor.c", dtype=torch.float32, shape=(F,), device=dev, gpu=False)
        _req(self.A, "Predictor.A")
        return self

    @property
    def d(self) -> int:
        return self.A.shape[1]

    @property
    def F(self) -> int:
        return self.Q.shape[0]

    def struct(self) -> _Predictor:
        self.check()
        r, d = self.A.shape
        return _Predictor(d, self.Q.shape[0], r, _dt(self.A), self.A.data_ptr(), self.Q.data_ptr(),
                          self.c.data_ptr())


@dataclass
class FFN:
    """FFN weights of one layer, neuron-major.  Dense: w_* [F][d] fp32/fp16.  4-bit: w_* uint8
    [F][d/2] with s_* fp16 [F][d/128].  Biases fp32 or None."""
    act: str
    w_up: torch.Tensor
    w_dT: torch.Tensor
    w_gate: Optional[torch.Tensor] = None
    s_up: Optional[torch.Tensor] = None
    s_gate: Optional[torch.Tensor] = None
    s_dT: Optional[torch.Tensor] = None
    b_up: Optional[torch.Tensor] = None
    b_gate: Optional[torch.Tensor] = None
    b_down: Optional[torch.Tensor] = None

    @property
    def d(self) -> int:
        return self.w_up.shape[1] * (2 if self.w_up.dtype == torch.uint8 else 1)

    @property
    def F(self) -> int:
        return self.w_up.shape[0]

    def check(self) -> "FFN":
        if self.act not in ("relu", "swiglu"):
            raise ValueError("FFN: act must be 'relu' or 'swiglu', got %r" % (self.act,))
        if self.w_up.dim() != 2:
            raise ValueError("FFN: w_up must be [F][d] (or uint8 [F][d/2])")
        dt = _dt(self.w_up)
        dev = self.w_up.device
        shp = tuple(self.w_up.shape)
        F, d = self.F, self.d
        _req(self.w_up, "FFN.w_up", device=dev, gpu=False)
        _req(self.w_dT, "FFN.w_dT", dtype=self.w_up.dtype, shape=shp, device=dev, gpu=False)
        if self.act == "swiglu":
            _req(self.w_gate, "FFN.w_gate", dtype=self.w_up.dtype, shape=shp, device=dev, gpu=False)
        if dt == PSFFN_I4G128:
            if d % 128:
                raise ValueError("FFN: 4-bit rows need d % 128 == 0")
            sshape = (F, d // 128)
            _req(self.s_up, "FFN.s_up", dtype=torch.float16, shape=sshape, device=dev, gpu=False)
            _req(self.s_dT, "FFN.s_dT", dtype=torch.float16, shape=sshape, device=dev, gpu=False)
            if self.act == "swiglu":
                _req(self.s_gate, "FFN.s_gate", dtype=torch.float16, shape=sshape, device=dev, gpu=False)
        for name in ("b_up", "b_gate"):
            t = getattr(self, name)
            if t is not None:
                _req(t, "FFN." + name, dtype=torch.float32, shape=(F,), device=dev, gpu=False)
        if self.b_down is not None:
            _req(self.b_down, "FFN.b_down", dtype=torch.float32, shape=(d,), device=dev, gpu=False)
        _req(self.w_up, "FFN.w_up")
        return self

    @property
    def act_dtype(self) -> torch.dtype:
        return _act_dtype(self.w_up.dtype)

    def struct(self) -> _FFN:
        self.check()
        p = lambda t: None if t is None else t.data_ptr()
        return _FFN(self.d, self.F, _dt(self.w_up), PSFFN_SWIGLU if self.act == "swiglu" else PSFFN_RELU,
                    p(self.w_up), p(self.w_gate), p(self.w_dT), p(self.s_up), p(self.s_gate), p(self.s_dT),
                    p(self.b_up), p(self.b_gate), p(self.b_down))

    def empty_like(self) -> "FFN":
        e = lambda t: None if t is None else torch.empty_like(t)
        return replace(self, w_up=e(self.w_up), w_dT=e(self.w_dT), w_gate=e(self.w_gate), s_up=e(self.s_up),
                       s_gate=e(self.s_gate), s_dT=e(self.s_dT), b_up=e(self.b_up), b_gate=e(self.b_gate))


def workspace_bytes(P: Optional[Predictor], W: Optional[FFN], B: int) -> int:
    ps = ctypes.byref(P.struct()) if P is not None else None
    ws = ctypes.byref(W.struct()) if W is not None else None
    n = _lib.psffn_workspace_bytes(ps, ws, int(B))
    if n == 0:
        raise PsffnError(PSFFN_E_INVALID_ARG, "workspace_bytes")
    return n


def workspace_init(ws: torch.Tensor, stream=None):
    _req(ws, "ws", dtype=torch.uint8)
    _check(_lib.psffn_workspace_init(_ptr(ws), ws.numel() * ws.element_size(), _stream(stream)), "workspace_init")


def new_workspace(P: Optional[Predictor], W: Optional[FFN], B: int, device="cuda", stream=None) -> torch.Tensor:
    n = (workspace_bytes(P, W, B) + 255) // 256 * 256
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    workspace_init(ws, stream)
    return ws


def _pair(P: Predictor, W: FFN):
    if P.F != W.F or P.d != W.d:
        raise ValueError("predictor (F %d, d %d) and FFN (F %d, d %d) describe different layers" % (P.F, P.d, W.F, W.d))
    if P.A.device != W.w_up.device:
        raise ValueError("predictor and FFN weights are on different devices")


def predict(P: Predictor, x: torch.Tensor, ws: torch.Tensor, thr: float = 0.0, idx: torch.Tensor = None,
            count: torch.Tensor = None, logits: torch.Tensor = None, stream=None, n_hot: int = 0):
    """Active neurons of the batch x [B][d]: (idx int32 [F] ascending, count int32 [1]) on the device.

    n_hot > 0: the first n_hot neurons of a hot-first layer are listed without prediction
    (psffn_predict_hot)."""
    s = P.struct()
    F = P.F
    B = _batch(x, P.d, _act_dtype(P.A.dtype))
    _req(x, "x", device=P.A.device)
    _outs(x.device, F, idx, count, logits, B, ws=ws)
    if idx is None:
        idx = torch.empty(F, dtype=torch.int32, device=x.device)
    if count is None:
        count = torch.empty(1, dtype=torch.int32, device=x.device)
    if n_hot:
        _check(_lib.psffn_predict_hot(ctypes.byref(s), int(n_hot), _ptr(x), B, float(thr), _ptr(idx), _ptr(count),
                                      _ptr(logits), _ptr(ws), ws.numel(), _stream(stream)), "predict_hot")
        return idx, count
    _check(_lib.psffn_predict(ctypes.byref(s), _ptr(x), B, float(thr), _ptr(idx), _ptr(count), _ptr(logits), _ptr(ws),
                              ws.numel(), _stream(stream)), "predict")
    return idx, count


def compact(logits: torch.Tensor, ws: torch.Tensor, thr: float = 0.0, idx=None, count=None, stream=None):
    if not isinstance(logits, torch.Tensor) or logits.dim() != 2:
        raise ValueError("logits: expected a [B][F] tensor")
    B, F = logits.shape
    _req(logits, "logits", dtype=torch.float32)
    _outs(logits.device, F, idx, count, ws=ws)
    if idx is None:
        idx = torch.empty(F, dtype=torch.int32, device=logits.device)
    if count is None:
        count = torch.empty(1, dtype=torch.int32, device=logits.device)
    _check(_lib.psffn_compact(_ptr(logits), B, F, float(thr), _ptr(idx), _ptr(count), _ptr(ws), ws.numel(),
                              _stream(stream)), "compact")
    return idx, count


def sparse_ffn(W: FFN, x: torch.Tensor, idx: torch.Tensor, count: torch.Tensor, ws: torch.Tensor,
               y: torch.Tensor = None, accumulate: bool = False, stream=None) -> torch.Tensor:
    s = W.struct()
    B = _batch(x, W.d, W.act_dtype)
    _req(x, "x", device=W.w_up.device)
    _req(idx, "idx", dtype=torch.int32, min_numel=1, device=x.device)
    _req(count, "count", dtype=torch.int32, min_numel=1, device=x.device)
    _outs(x.device, 1, None, None, B=B, y=y, d=W.d, ws=ws)
    if y is None:
        y = torch.empty(B, W.d, dtype=torch.float32, device=x.device)
    _check(_lib.psffn_sparse_ffn(ctypes.byref(s), _ptr(x), B, _ptr(idx), _ptr(count), _ptr(y), int(bool(accumulate)),
                                 _ptr(ws), ws.numel(), _stream(stream)), "sparse_ffn")
    return y


def layer(P: Predictor, W: FFN, x: torch.Tensor, ws: torch.Tensor, thr: float = 0.0, idx: torch.Tensor = None,
          count: torch.Tensor = None, logits: torch.Tensor = None, y: torch.Tensor = None, accumulate: bool = False,
          stream=None, n_hot: int = 0):
    """One decode step of one layer (predict + sparse FFN in one call): returns (idx, count, y).

    n_hot > 0: hot prefix as in predict (psffn_layer_hot)."""
    sp, sw = P.struct(), W.struct()
    _pair(P, W)
    F = P.F
    B = _batch(x, W.d, W.act_dtype)
    _req(x, "x", device=W.w_up.device)
    _outs(x.device, F, idx, count, logits, B, y, W.d, ws)
    if idx is None:
        idx = torch.empty(F, dtype=torch.int32, device=x.device)
    if count is None:
        count = torch.empty(1, dtype=torch.int32, device=x.device)
    if y is None:
        y = torch.empty(B, W.d, dtype=torch.float32, device=x.device)
    if n_hot:
        _check(_lib.psffn_layer_hot(ctypes.byref(sp), ctypes.byref(sw), int(n_hot), _ptr(x), B, float(thr), _ptr(idx),
                                    _ptr(count), _ptr(logits), _ptr(y), int(bool(accumulate)), _ptr(ws), ws.numel(),
                                    _stream(stream)), "layer_hot")
        return idx, count, y
    _check(_lib.psffn_layer(ctypes.byref(sp), ctypes.byref(sw), _ptr(x), B, float(thr), _ptr(idx), _ptr(count),
                            _ptr(logits), _ptr(y), int(bool(accumulate)), _ptr(ws), ws.numel(), _stream(stream)),
           "layer")
    return idx, count, y


def layer_noalloc(P: Predictor, W: FFN, x: torch.Tensor, thr: float = 0.0, idx: torch.Tensor = None,
                  count: torch.Tensor = None, logits: torch.Tensor = None, y: torch.Tensor = None,
                  accumulate: bool = False, stream=None):
    """psffn_layer with the library's static per-GPU scratch instead of a workspace (no allocation
    in the library; calls overlapping on one GPU race).  Returns (idx, count, y)."""
    sp, sw = P.struct(), W.struct()
    _pair(P, W)
    F = P.F
    B = _batch(x, W.d, W.act_dtype)
    _req(x, "x", device=W.w_up.device)
    _outs(x.device, F, idx, count, logits, B, y, W.d)
    if idx is None:
        idx = torch.empty(F, dtype=torch.int32, device=x.device)
    if count is None:
        count = torch.empty(1, dtype=torch.int32, device=x.device)
    if y is None:
        y = torch.empty(B, W.d, dtype=torch.float32, device=x.device)
    _check(_lib.psffn_layer_noalloc(ctypes.byref(sp), ctypes.byref(sw), _ptr(x), B, float(thr), _ptr(idx),
                                    _ptr(count), _ptr(logits), _ptr(y), int(bool(accumulate)), _stream(stream)),
           "layer_noalloc")
    return idx, count, y


def layer_ln(P: Predictor, W: FFN, x: torch.Tensor, ws: torch.Tensor, eps: float = 1e-5, h: torch.Tensor = None,
             thr: float = 0.0, idx: torch.Tensor = None, count: torch.Tensor = None, logits: torch.Tensor = None,
             stream=None):
    """One decode-stack step on the fp32 residual x [B][d], in place: h = fp16(LayerNorm(x)), then
    x += the sparse FFN of h (psffn_layer_ln).  Returns (idx, count, h)."""
    sp, sw = P.struct(), W.struct()
    _pair(P, W)
    F, d = P.F, W.d
    B = _batch(x, d, torch.float32)
    _req(x, "x", device=W.w_up.device)
    if h is not None:
        _req(h, "h", dtype=torch.float16, shape=(B, d), device=x.device)
    _outs(x.device, F, idx, count, logits, B, ws=ws)
    if idx is None:
        idx = torch.empty(F, dtype=torch.int32, device=x.device)
    if count is None:
        count = torch.empty(1, dtype=torch.int32, device=x.device)
    if h is None:
        h = torch.empty(B, d, dtype=torch.float16, device=x.device)
    _check(_lib.psffn_layer_ln(ctypes.byref(sp), ctypes.byref(sw), _ptr(x), float(eps), _ptr(h), B, float(thr),
                               _ptr(idx), _ptr(count), _ptr(logits), _ptr(ws), ws.numel(), _stream(stream)),
           "layer_ln")
    return idx, count, h


def profile_counts(W: FFN, X: torch.Tensor, counts: torch.Tensor = None, stream=None) -> torch.Tensor:
    s = W.struct()
    if not isinstance(X, torch.Tensor) or X.dim() != 2 or X.shape[0] < 1:
        raise ValueError("X: expected a [T][d] tensor with T >= 1")
    _req(X, "X", dtype=W.act_dtype, shape=(X.shape[0], W.d), device=W.w_up.device)
    if counts is not None:
        _req(counts, "counts", dtype=torch.int32, shape=(W.F,), device=X.device)
    if counts is None:
        counts = torch.empty(W.F, dtype=torch.int32, device=X.device)
    _check(_lib.psffn_profile_counts(ctypes.byref(s), _ptr(X), X.shape[0], _ptr(counts), _stream(stream)),
           "profile_counts")
    return counts


def permute_hot_first(counts: torch.Tensor, W: Optional[FFN] = None, P: Optional[Predictor] = None,
                      stream=None):
    """Returns (perm, W', P'): W' and P' are new buffers holding the hot-first reordering."""
    if not isinstance(counts, torch.Tensor) or counts.dim() != 1:
        raise ValueError("counts: expected an int32 [F] tensor")
    F = counts.shape[0]
    _req(counts, "counts", dtype=torch.int32)
    for M in (W, P):
        if M is not None:
            M.check()
            if M.F != F:
                raise ValueError("permute_hot_first: counts has %d entries, the layer %d neurons" % (F, M.F))
    perm = torch.empty(F, dtype=torch.int32, device=counts.device)
    Wd = W.empty_like() if W is not None else None
    Pd = Predictor(P.A, torch.empty_like(P.Q), torch.empty_like(P.c)) if P is not None else None
    sW, dW = (W.struct(), Wd.struct()) if W is not None else (None, None)
    sP, dP = (P.struct(), Pd.struct()) if P is not None else (None, None)
    ref = lambda v: ctypes.byref(v) if v is not None else None
    _check(_lib.psffn_permute_hot_first(_ptr(counts), F, _ptr(perm), ref(sW), ref(dW), ref(sP), ref(dP),
                                        _stream(stream)), "permute_hot_first")
    if Wd is not None and W.b_down is not None:
        Wd.b_down = W.b_down
    return perm, Wd, Pd


def layernorm_f16(x: torch.Tensor, eps: float = 1e-5, out: torch.Tensor = None, stream=None) -> torch.Tensor:
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError("x: expected a float32 [B][d] tensor")
    B, d = x.shape
    _req(x, "x", dtype=torch.float32)
    if out is not None:
        _req(out, "out", dtype=torch.float16, shape=(B, d), device=x.device)
    if out is None:
        out = torch.empty(B, d, dtype=torch.float16, device=x.device)
    _check(_lib.psffn_layernorm_f16(_ptr(x), B, d, float(eps), _ptr(out), _stream(stream)), "layernorm_f16")
    return out
