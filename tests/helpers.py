"""Shared helpers of the GPU parity tests: descriptors for both sides built from one synthetic
layer, and the comparison rules.

Comparison rules (parity bar):
  * active sets: bit-exact, except neurons whose oracle logit (max over the batch) lies within
    BAND = 1e-6 of the threshold, where fp32 and fp64 accumulation may legitimately disagree;
  * FFN outputs: ||y - y_ref||_inf / ||y_ref||_inf <= 1e-5 for fp32 weights, 2e-3 for fp16 and
    4-bit weights (fp32 accumulation); y_ref == 0 requires y == 0 exactly;
  * integer and index outputs (counts, permutation, compaction of given logits): bit-exact.
Oracle inputs only ever come from the synthetic generator or the oracle itself.
"""
from dataclasses import replace

import numpy as np
import torch

import oracle
import synth

BAND = 1e-6


def tol_for(storage: str) -> float:
    return 1e-5 if storage == "f32" else 2e-3


def ffn_of(L, ps):
    return ps.FFN(L.spec.act, L.w_up, L.w_dT, w_gate=L.w_gate, s_up=L.s_up, s_gate=L.s_gate, s_dT=L.s_dT, b_up=L.b_up,
                  b_gate=L.b_gate, b_down=L.b_down)


def pred_of(L, ps):
    return ps.Predictor(L.A, L.Q, L.c)


def oracle_layer(n: dict, act: str, b_down=None):
    return oracle.Layer(act, n["w_up"], n["w_dT"], w_gate=n["w_gate"], s_up=n["s_up"], s_gate=n["s_gate"],
                        s_dT=n["s_dT"], b_up=n["b_up"], b_gate=n["b_gate"],
                        b_down=n["b_down"] if b_down is None else b_down)


def spec_variant(name: str, **kw):
    return replace(synth.CONFIGS[name], **kw)


def check_set(idx, count, logits_ref, thr=0.0, n_hot=0):
    """GPU list (idx tensor, count tensor) against oracle logits [B][F]; returns stats.
    n_hot: the first n_hot neurons must be listed whatever their logits."""
    F = logits_ref.shape[1]
    n = int(count.cpu()[0])
    assert 0 <= n <= F
    got_idx = idx[:n].cpu().numpy()
    assert np.all(np.diff(got_idx) > 0), "list not strictly ascending"
    assert n == 0 or (got_idx[0] >= 0 and got_idx[-1] < F)
    m = logits_ref.max(axis=0)
    hot = np.arange(F) < n_hot
    ref = (m > thr) | hot
    near = (np.abs(m - thr) < BAND) & ~hot
    got = np.zeros(F, dtype=bool)
    got[got_idx] = True
    bad = (got != ref) & ~near
    assert not bad.any(), "active-set mismatch outside the band at neurons %s (logits %s)" % (
        np.flatnonzero(bad)[:8], m[bad][:8])
    return {"count": n, "ref_count": int(ref.sum()), "in_band_diff": int(((got != ref) & near).sum()),
            "exact": bool((got == ref).all())}


def rel_inf(y, ref) -> float:
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.abs(ref).max() if ref.size else 0.0
    if den == 0.0:
        return 0.0 if np.all(y == 0) else float("inf")
    return float(np.abs(y - ref).max() / den)


def check_y(y, ref, tol):
    e = rel_inf(y, ref)
    assert e <= tol, "max relative error %.3e > %.1e" % (e, tol)
    return e


def ln_bound(x, ref):
    """Allowed |LN_gpu - LN_ref| per element (fp16 output of an fp32 LayerNorm against the fp64
    oracle): one fp16 ulp of the result, plus what fp32 arithmetic cannot avoid near zero -- x - mean
    rounds at eps32 (|x| + |mean|), divided by the row's sigma (a few roundings: factor 16)."""
    x = np.asarray(x, dtype=np.float64)
    ulp = np.spacing(np.abs(ref).astype(np.float16)).astype(np.float64)
    eps32 = float(np.finfo(np.float32).eps)
    slack = 16 * eps32 * (np.abs(x).max(axis=1) + np.abs(x.mean(axis=1))) / np.sqrt(x.var(axis=1) + 1e-5)
    return ulp + slack[:, None]


def dequant_rows(n: dict, name: str, d: int):
    """The stored rows of w_<name> as float64 (4-bit rows decoded by the oracle's own decoder)."""
    w = n["w_" + name]
    if w.dtype == np.uint8:
        return oracle.i4_dequant(w, n["s_" + name], d)
    return w.astype(np.float64)


def check_counts(got, orc, n: dict, X):
    """GPU fire counts against the oracle's deciding pre-activations z (fp64).  The GPU forms each z
    in fp32 from exact products (fp16 x fp16, 4-bit x fp16; fp32 products round once), summed per
    lane over d/64 slices of the row and then over a 6-level butterfly, plus the bias: a summation
    tree of depth at most k = d/64 + 8, so |z_gpu - z| <= gamma_k * (sum_k |w_k x_k| + |b|) with
    gamma_k = k u / (1 - k u), u = 2^-24.  A token whose z lies within that margin of zero may count
    either way; the count must lie between the two extremes, and equal the oracle's count for every
    neuron with no such token.  Returns the number of neurons with an ambiguous token."""
    X = np.asarray(X)
    d = orc.d
    branch = "up" if orc.act == oracle.RELU else "gate"
    Wd = dequant_rows(n, branch, d)
    bias = n["b_" + branch]
    bias = np.zeros(orc.F) if bias is None else bias.astype(np.float64)
    S = np.abs(Wd) @ np.abs(X.astype(np.float64)).T + np.abs(bias)[:, None]  # [F][T]
    k = d / 64 + 8
    u = 2.0 ** -24
    margin = (k * u / (1 - k * u)) * S
    z = orc.pre_activations(X).T  # [F][T]
    lo = (z > margin).sum(axis=1)
    hi = (z > -margin).sum(axis=1)
    got = np.asarray(got)
    assert np.all(lo <= got) and np.all(got <= hi), "fire counts outside the fp32-accumulation bracket"
    exact = lo == hi
    assert np.array_equal(got[exact], (z > 0).sum(axis=1)[exact])
    return int((~exact).sum())
