"""CPU oracle for the predictor-gated sparse FFN -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this package.  The product library never links, loads or calls it, and it shares no
code with the HIP path: the arithmetic lives in ``psffn_oracle.c`` (scalar fp64 loops over the
stored bytes), this module only marshals numpy arrays into it and composes its steps.

Method, as the pages fix it ("PowerInfer: Fast Large Language Model Serving with a
Consumer-grade GPU", Elamur Research summary):
  * Summary, 2nd paragraph -- lightweight per-layer predictors guess which MLP neurons fire,
    neuron-level kernels compute only those and skip the rest; neurons are profiled offline.
  * Interesting ideas, I4 -- the kernels act directly on weight rows and columns.
  * Interesting ideas, I1 -- the most used neurons are placed first (fastest memory).
  * Key points (sparsity) -- ReLU FFNs (OPT) are ~97% sparse, SwiGLU ones (LLaMA2) ~43%.

Readings where the pages are silent (each also listed in the design notes):
  * predictor = linear low rank, l = Q (A x) + c; fire <=> sigmoid(l) > 1/2 <=> l > 0;
  * a batch shares the union of its tokens' predicted sets, listed in ascending order;
  * SwiGLU output a = silu(gate) * up, active set predicted from the gate branch;
  * 4-bit weights: signed nibbles, low nibble first, one fp16 scale per 128 elements;
  * hot-first order: descending profiled fire count, ties by ascending index;
  * decode stack: x <- x + FFN(fp16(LayerNorm(x))), gamma 1, beta 0, eps 1e-5.

Every function is pinned by the ``not gpu`` tests in ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "psffn_oracle.c")
_LIB = os.path.join(_HERE, "_psffn_oracle.so")
# a separately built copy of the same source (the host-sanitizer test builds one with ASan + UBSan)
_LIB_OVERRIDE = os.environ.get("PSFFN_ORACLE_LIB")

F32, F16, I4G128 = 0, 1, 2
RELU, SWIGLU = 0, 1


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (plain IEEE fp64: no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-shared", "-fPIC",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _L():
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(_LIB_OVERRIDE if _LIB_OVERRIDE else build())
        _p, _i, _d = ctypes.c_void_p, ctypes.c_int, ctypes.c_double
        _lib.orc_half_to_double.restype = _d
        _lib.orc_half_to_double.argtypes = [ctypes.c_uint16]
        _lib.orc_double_to_half.restype = ctypes.c_uint16
        _lib.orc_double_to_half.argtypes = [_d]
        _lib.orc_i4_elem.restype = _d
        _lib.orc_i4_elem.argtypes = [_p, _p, ctypes.c_size_t, ctypes.c_size_t, ctypes.c_size_t]
        _lib.orc_predict_logits.restype = None
        _lib.orc_predict_logits.argtypes = [_i, _p, _p, _p, _i, _i, _i, _i, _p, _i, _p]
        _lib.orc_compact.restype = _i
        _lib.orc_compact.argtypes = [_p, _i, _i, _d, _p]
        _lib.orc_compact_hot.restype = _i
        _lib.orc_compact_hot.argtypes = [_p, _i, _i, _d, _i, _p]
        _lib.orc_activations.restype = None
        _lib.orc_activations.argtypes = [_i, _i, _i, _p, _p, _p, _p, _p, _p, _i, _p, _i, _p, _i, _p]
        _lib.orc_sparse_ffn.restype = None
        _lib.orc_sparse_ffn.argtypes = [_i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p, _p, _i, _p, _i, _p, _i, _p]
        _lib.orc_fire_counts.restype = None
        _lib.orc_fire_counts.argtypes = [_i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _i, _p, _i, _d, _p]
        _lib.orc_pre_activations.restype = None
        _lib.orc_pre_activations.argtypes = [_i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _i, _p, _i, _p]
        _lib.orc_hot_first_perm.restype = None
        _lib.orc_hot_first_perm.argtypes = [_p, _i, _p]
        _lib.orc_layernorm.restype = None
        _lib.orc_layernorm.argtypes = [_p, _i, _i, _d, _p]
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    """Contiguous numpy view of an array (or None) with the exact storage dtype required."""
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError("oracle: expected %s, got %s" % (np.dtype(dtype), a.dtype))
    return a


def _dense_code(a):
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.float16:
        return F16
    raise TypeError("oracle: dense operand must be float32 or float16, got %s" % a.dtype)


# ---------------------------------------------------------------------------------------------
# elementary decoders (pinned against numpy's float16 and hand-worked bytes)

def half_to_double(bits: int) -> float:
    return _L().orc_half_to_double(int(bits) & 0xFFFF)


def double_to_half_bits(v: float) -> int:
    return int(_L().orc_double_to_half(float(v)))


def round_to_f16(v: np.ndarray) -> np.ndarray:
    """Round every element of a float64 array to fp16 (RNE) with the oracle's own encoder."""
    flat = np.asarray(v, dtype=np.float64).ravel()
    out = np.empty(flat.shape, dtype=np.uint16)
    f = _L().orc_double_to_half
    for k, x in enumerate(flat):
        out[k] = f(float(x))
    return out.view(np.float16).reshape(np.shape(v))


def i4_dequant(packed: np.ndarray, scales: np.ndarray, d: int) -> np.ndarray:
    """Decode a whole 4-bit matrix [rows][d] element by element (float64)."""
    packed = _c(packed, np.uint8)
    scales = _c(scales, np.float16)
    rows = packed.shape[0]
    f = _L().orc_i4_elem
    out = np.empty((rows, d), dtype=np.float64)
    pp, sp = _ptr(packed), _ptr(scales)
    for i in range(rows):
        for j in range(d):
            out[i, j] = f(pp, sp, d, i, j)
    return out


# ---------------------------------------------------------------------------------------------
# the method's steps

def predict_logits(A, Q, c, x):
    """Logits [B][F] (float64) of the low-rank predictor l = Q (A x) + c for each row of x."""
    A = np.ascontiguousarray(A)
    Q = np.ascontiguousarray(Q)
    dt_p = _dense_code(A)
    if Q.dtype != A.dtype:
        raise TypeError("oracle: A and Q must share a dtype")
    x = np.ascontiguousarray(np.atleast_2d(x))
    dt_x = _dense_code(x)
    c = _c(c, np.float32)
    r, d = A.shape
    F = Q.shape[0]
    B = x.shape[0]
    assert Q.shape == (F, r) and x.shape == (B, d) and c.shape == (F,)
    out = np.empty((B, F), dtype=np.float64)
    _L().orc_predict_logits(dt_p, _ptr(A), _ptr(Q), _ptr(c), d, r, F, dt_x, _ptr(x), B, _ptr(out))
    return out


def compact(logits, thr: float = 0.0, n_hot: int = 0):
    """Ascending int32 list of neurons whose logit exceeds thr for at least one token.

    n_hot > 0: the hot prefix [0, n_hot) of a hot-first layer is kept whatever its logits (the
    predictor gates only the cold tail)."""
    logits = np.ascontiguousarray(np.atleast_2d(logits), dtype=np.float64)
    B, F = logits.shape
    idx = np.empty(F, dtype=np.int32)
    if n_hot:
        n = _L().orc_compact_hot(_ptr(logits), B, F, float(thr), int(n_hot), _ptr(idx))
    else:
        n = _L().orc_compact(_ptr(logits), B, F, float(thr), _ptr(idx))
    return idx[:n].copy()


class Layer:
    """The stored bytes of one FFN layer, neuron-major (row i of each matrix is neuron i).

    dense storage: w_up, w_gate, w_dT are float32/float16 [F][d], scales None.
    4-bit storage: w_* are uint8 [F][d/2], s_* float16 [F][d/128].
    Biases are float32 [F] (b_up, b_gate) and [d] (b_down), or None for zero.
    """

    def __init__(self, act, w_up, w_dT, w_gate=None, s_up=None, s_gate=None, s_dT=None,
                 b_up=None, b_gate=None, b_down=None):
        self.act = RELU if act in (RELU, "relu") else SWIGLU
        if w_up.dtype == np.uint8:
            self.dt = I4G128
            self.d = w_up.shape[1] * 2
            cast = lambda a: _c(a, np.uint8)
            self.s_up, self.s_gate, self.s_dT = (_c(s, np.float16) for s in (s_up, s_gate, s_dT))
        else:
            self.dt = _dense_code(w_up)
            self.d = w_up.shape[1]
            cast = lambda a: _c(a, w_up.dtype)
            self.s_up = self.s_gate = self.s_dT = None
        self.F = w_up.shape[0]
        self.w_up, self.w_dT = cast(w_up), cast(w_dT)
        self.w_gate = cast(w_gate) if w_gate is not None else None
        if self.act == SWIGLU and self.w_gate is None:
            raise ValueError("oracle: SwiGLU needs w_gate")
        self.b_up, self.b_gate, self.b_down = (_c(b, np.float32) for b in (b_up, b_gate, b_down))

    def _wargs(self):
        return (self.dt, self.act, self.d)

    def activations(self, x, idx):
        x = np.ascontiguousarray(np.atleast_2d(x))
        idx = _c(idx, np.int32)
        B = x.shape[0]
        a = np.empty((len(idx), B), dtype=np.float64)
        _L().orc_activations(self.dt, self.act, self.d, _ptr(self.w_up), _ptr(self.s_up), _ptr(self.w_gate),
                             _ptr(self.s_gate), _ptr(self.b_up), _ptr(self.b_gate), _dense_code(x), _ptr(x), B,
                             _ptr(idx), len(idx), _ptr(a))
        return a

    def sparse_ffn(self, x, idx):
        """y [B][d] (float64) computed over the listed neurons only."""
        x = np.ascontiguousarray(np.atleast_2d(x))
        idx = _c(idx, np.int32)
        B = x.shape[0]
        assert x.shape[1] == self.d
        y = np.empty((B, self.d), dtype=np.float64)
        _L().orc_sparse_ffn(self.dt, self.act, self.d, self.F, _ptr(self.w_up), _ptr(self.s_up), _ptr(self.w_gate),
                            _ptr(self.s_gate), _ptr(self.w_dT), _ptr(self.s_dT), _ptr(self.b_up), _ptr(self.b_gate),
                            _ptr(self.b_down), _dense_code(x), _ptr(x), B, _ptr(idx), len(idx), _ptr(y))
        return y

    def dense_ffn(self, x):
        return self.sparse_ffn(x, np.arange(self.F, dtype=np.int32))

    def fire_counts(self, X, thr: float = 0.0):
        """counts[i] = number of tokens of X whose deciding pre-activation of neuron i exceeds thr
        (the profile is thr = 0)."""
        X = np.ascontiguousarray(np.atleast_2d(X))
        counts = np.empty(self.F, dtype=np.int32)
        _L().orc_fire_counts(self.dt, self.act, self.d, self.F, _ptr(self.w_up), _ptr(self.s_up), _ptr(self.w_gate),
                             _ptr(self.s_gate), _ptr(self.b_up), _ptr(self.b_gate), _dense_code(X), _ptr(X),
                             X.shape[0], float(thr), _ptr(counts))
        return counts

    def pre_activations(self, X):
        """z [T][F] (float64): the deciding pre-activation of every neuron on every token (ReLU: up,
        SwiGLU: gate), the quantity whose sign fire_counts counts."""
        X = np.ascontiguousarray(np.atleast_2d(X))
        T = X.shape[0]
        z = np.empty((T, self.F), dtype=np.float64)
        _L().orc_pre_activations(self.dt, self.act, self.d, self.F, _ptr(self.w_up), _ptr(self.s_up),
                                 _ptr(self.w_gate), _ptr(self.s_gate), _ptr(self.b_up), _ptr(self.b_gate),
                                 _dense_code(X), _ptr(X), T, _ptr(z))
        return z

    def permuted(self, perm):
        """The same layer with its neurons reordered: new neuron k = old neuron perm[k]."""
        g = lambda a: None if a is None else np.ascontiguousarray(a[perm])
        return Layer(self.act, g(self.w_up), g(self.w_dT), w_gate=g(self.w_gate), s_up=g(self.s_up),
                     s_gate=g(self.s_gate), s_dT=g(self.s_dT), b_up=g(self.b_up), b_gate=g(self.b_gate),
                     b_down=self.b_down)


def hot_first_perm(counts):
    counts = _c(counts, np.int32)
    perm = np.empty(len(counts), dtype=np.int32)
    _L().orc_hot_first_perm(_ptr(counts), len(counts), _ptr(perm))
    return perm


def layernorm(x, eps: float = 1e-5):
    x = _c(np.atleast_2d(x), np.float32)
    B, d = x.shape
    out = np.empty((B, d), dtype=np.float64)
    _L().orc_layernorm(_ptr(x), B, d, float(eps), _ptr(out))
    return out


def predicted_layer(A, Q, c, layer: Layer, x, thr: float = 0.0):
    """One decode step of one layer: predict, keep the union set, compute the FFN over it.
    Returns (idx, logits, y)."""
    logits = predict_logits(A, Q, c, x)
    idx = compact(logits, thr)
    return idx, logits, layer.sparse_ffn(x, idx)


def stack_step(layers, x, thr: float = 0.0, eps: float = 1e-5):
    """Decode stack: for each (A, Q, c, Layer) in order, x <- x + FFN(fp16(LayerNorm(x))), with
    the FFN restricted to the predicted union set.  x is the fp32 residual [B][d]; the residual
    is kept in fp32 between layers.  Returns the new residual (float32)."""
    x = np.ascontiguousarray(np.atleast_2d(x), dtype=np.float32)
    for (A, Q, c, layer) in layers:
        h = round_to_f16(layernorm(x, eps))
        _, _, y = predicted_layer(A, Q, c, layer, h, thr)
        x = (x.astype(np.float64) + y).astype(np.float32)
    return x
