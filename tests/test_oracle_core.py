"""Pins for the CPU oracle: every routine is checked against something other than itself --
library routines (numpy fp64 matmul, numpy's float16, torch's layer_norm, Python's sort),
closed forms, invariants and hand-worked fixtures in tests/golden/."""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(12345)


def _read_kv(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if "=" in line:
                k, v = line.split("=")
                out[k.strip()] = np.array([float(t) for t in v.split()])
    return out


# ------------------------------------------------------------------ elementary decoders

def test_half_decoder_matches_numpy_on_every_bit_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.half_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros keep their sign
    assert math.copysign(1.0, oracle.half_to_double(0x8000)) == -1.0


def test_half_encoder_round_to_nearest_even_matches_numpy():
    vals = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 5, 20000),
        # exact halfway points between neighbouring halves (ties must go to even)
        (np.arange(0, 4000, dtype=np.uint16).view(np.float16).astype(np.float64)
         + np.arange(1, 4001, dtype=np.uint16).view(np.float16).astype(np.float64)) / 2,
        [0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e6, -1e6, 2.0 ** -24, 2.0 ** -25, 2.0 ** -25 * 1.0001,
         2.0 ** -14, 2.0 ** -14 * (1 - 2.0 ** -12)],
    ])
    got = oracle.round_to_f16(vals)
    with np.errstate(over="ignore"):
        ref = vals.astype(np.float16)
    assert np.array_equal(got.view(np.uint16), ref.view(np.uint16))


def test_int4_hand_worked_bytes():
    with open(os.path.join(GOLDEN, "int4_worked.txt")) as f:
        rows = [l.split("#")[0].split() for l in f if l.strip() and not l.startswith("#")]
    assert len(rows) == 10
    d = 256
    for byte, col, scale, want in rows:
        packed = np.zeros((1, d // 2), dtype=np.uint8)
        scales = np.zeros((1, d // 128), dtype=np.float16)
        # put the byte at byte 70 (group 1: elements 140, 141) to exercise the group index
        packed[0, 70] = int(byte, 16)
        scales[0, 1] = np.float16(float(scale))
        deq = oracle.i4_dequant(packed, scales, d)
        assert deq[0, 140 + int(col)] == float(want)
        others = np.delete(deq[0], [140, 141])  # every other byte is zero
        assert np.all(others == 0.0)


def test_int4_roundtrip_against_independent_encoder():
    # The encoder lives in the input generator; the decoder in the oracle.  Their round trip must
    # reproduce the encoder's exact q*s values, and q*s must be within s/2 of the original weight.
    g = torch.Generator().manual_seed(7)
    w = torch.randn(6, 512, generator=g) / math.sqrt(512)
    packed, s16, exact = synth.quantize_i4_g128(w)
    deq = oracle.i4_dequant(packed.numpy(), s16.numpy(), 512)
    assert np.array_equal(deq, exact.numpy())
    s = np.repeat(s16.numpy().astype(np.float64), 128, axis=1)
    assert np.all(np.abs(deq - w.double().numpy()) <= s / 2 * (1 + 1e-6) + 1e-12)
    # multiples k*s (k in [-7, 7]) survive exactly
    ks = torch.tensor([[-7, -3, 0, 1, 5, 7] * 2 + [0] * 116 + [7]], dtype=torch.float32)
    ks = ks[:, :128] * 0.125
    p2, s2, e2 = synth.quantize_i4_g128(ks)
    assert np.array_equal(oracle.i4_dequant(p2.numpy(), s2.numpy(), 128), ks.double().numpy())


# ------------------------------------------------------------------ predictor + compaction

def test_predictor_matches_numpy_fp64():
    for dt in (np.float32, np.float16):
        d, r, F, B = 96, 12, 70, 3
        A = (rng.standard_normal((r, d)) / 10).astype(dt)
        Q = (rng.standard_normal((F, r)) / 3).astype(dt)
        c = rng.standard_normal(F).astype(np.float32)
        x = rng.standard_normal((B, d)).astype(dt)
        got = oracle.predict_logits(A, Q, c, x)
        ref = (Q.astype(np.float64) @ (A.astype(np.float64) @ x.astype(np.float64).T)).T + c.astype(np.float64)
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_compact_is_flatnonzero_of_union_and_strict():
    logits = rng.standard_normal((4, 500))
    logits[:, 17] = 0.0  # exactly at threshold -> inactive (strict >)
    logits[2, 18] = 1e-300
    idx = oracle.compact(logits, 0.0)
    assert np.array_equal(idx, np.flatnonzero(logits.max(axis=0) > 0.0))
    assert 17 not in idx and 18 in idx
    assert idx.dtype == np.int32 and np.all(np.diff(idx) > 0)
    thr = 0.7
    assert np.array_equal(oracle.compact(logits, thr), np.flatnonzero(logits.max(axis=0) > thr))
    assert len(oracle.compact(np.full((1, 9), -1.0))) == 0
    assert len(oracle.compact(np.full((1, 9), 1.0))) == 9


def test_hand_worked_layer():
    g = _read_kv("ffn_worked.txt")
    f32 = lambda a, *s: np.asarray(a, dtype=np.float32).reshape(*s)
    x = f32(g["x"], 1, 2)
    A, Q, c = f32(g["A"], 1, 2), f32(g["Q"], 3, 1), f32(g["c"], 3)
    lay = oracle.Layer("relu", f32(g["W_up"], 3, 2), f32(g["W_dT"], 3, 2), b_up=f32(g["b_up"], 3))
    idx, logits, y = oracle.predicted_layer(A, Q, c, lay, x)
    assert np.array_equal(logits[0], g["logits"])
    assert np.array_equal(idx, g["kept"].astype(np.int32))
    assert np.array_equal(y[0], g["y_kept"])
    assert np.array_equal(lay.dense_ffn(x)[0], g["y_dense"])
    sw = oracle.Layer("swiglu", f32(g["W_up2"], 3, 2), f32(g["W_dT"], 3, 2), w_gate=f32(g["W_up"], 3, 2),
                      b_gate=f32(g["b_up"], 3))
    assert np.array_equal(sw.sparse_ffn(x, idx)[0], g["swiglu_y_kept"])
    np.testing.assert_allclose(sw.dense_ffn(x)[0], g["swiglu_y_dense"], rtol=0, atol=1e-9)


# ------------------------------------------------------------------ FFN over a neuron list

def _np_relu_ffn(Wu, bu, Wd, x, keep, bd=None):
    z = Wu.astype(np.float64) @ x.astype(np.float64) + bu.astype(np.float64)
    a = np.maximum(z, 0.0) * keep
    y = Wd.astype(np.float64).T @ a
    return y if bd is None else y + bd.astype(np.float64)


def _np_swiglu_ffn(Wg, bg, Wu, Wd, x, keep):
    g = Wg.astype(np.float64) @ x.astype(np.float64) + bg.astype(np.float64)
    u = Wu.astype(np.float64) @ x.astype(np.float64)
    a = g / (1.0 + np.exp(-g)) * u * keep
    return Wd.astype(np.float64).T @ a


@pytest.mark.parametrize("dt", [np.float32, np.float16])
def test_relu_ffn_brute_force_all_masks(dt):
    d, F = 6, 10
    Wu = rng.standard_normal((F, d)).astype(dt)
    Wd = rng.standard_normal((F, d)).astype(dt)
    bu = rng.standard_normal(F).astype(np.float32)
    bd = rng.standard_normal(d).astype(np.float32)
    x = rng.standard_normal((1, d)).astype(dt)
    lay = oracle.Layer("relu", Wu, Wd, b_up=bu, b_down=bd)
    for m in range(1 << F):
        keep = np.array([(m >> i) & 1 for i in range(F)], dtype=np.float64)
        idx = np.flatnonzero(keep).astype(np.int32)
        np.testing.assert_allclose(lay.sparse_ffn(x, idx)[0], _np_relu_ffn(Wu, bu, Wd, x[0], keep, bd),
                                   rtol=1e-12, atol=1e-12)


def test_swiglu_ffn_brute_force_all_masks():
    d, F = 5, 9
    Wg, Wu, Wd = (rng.standard_normal((F, d)).astype(np.float16) for _ in range(3))
    bg = rng.standard_normal(F).astype(np.float32)
    x = rng.standard_normal((1, d)).astype(np.float16)
    lay = oracle.Layer("swiglu", Wu, Wd, w_gate=Wg, b_gate=bg)
    for m in range(1 << F):
        keep = np.array([(m >> i) & 1 for i in range(F)], dtype=np.float64)
        idx = np.flatnonzero(keep).astype(np.int32)
        np.testing.assert_allclose(lay.sparse_ffn(x, idx)[0], _np_swiglu_ffn(Wg, bg, Wu, Wd, x[0], keep),
                                   rtol=1e-12, atol=1e-12)


def _small_layer(name, seed=3, d=128, F=256, r=16):
    spec = synth.CONFIGS[name]
    L = synth.make_layer(spec, seed=seed, d=d, F=F, r=r)
    n = L.numpy()
    lay = oracle.Layer(spec.act, n["w_up"], n["w_dT"], w_gate=n["w_gate"], s_up=n["s_up"], s_gate=n["s_gate"],
                       s_dT=n["s_dT"], b_up=n["b_up"], b_gate=n["b_gate"], b_down=n["b_down"])
    x = synth.make_tokens(spec, 8, seed=seed, d=d).numpy()
    return spec, L, n, lay, x


@pytest.mark.parametrize("name", ["tiny_relu_f32", "opt30b_relu_f16", "llama2_13b_swiglu_f16", "opt175b_relu_i4"])
def test_all_active_is_dense_and_empty_is_bias(name):
    spec, L, n, lay, x = _small_layer(name)
    F, d = lay.F, lay.d
    y_all = lay.sparse_ffn(x, np.arange(F, dtype=np.int32))
    # dense FFN written with numpy over the decoded weights
    if lay.dt == oracle.I4G128:
        dq = lambda w, s: oracle.i4_dequant(w, s, d)
        Wu, Wd = dq(n["w_up"], n["s_up"]), dq(n["w_dT"], n["s_dT"])
    else:
        Wu, Wd = n["w_up"].astype(np.float64), n["w_dT"].astype(np.float64)
    ones = np.ones(F)
    for b in range(x.shape[0]):
        if spec.act == "relu":
            ref = _np_relu_ffn(Wu, n["b_up"], Wd, x[b], ones)
        else:
            ref = _np_swiglu_ffn(n["w_gate"], n["b_gate"], Wu, Wd, x[b], ones)
        np.testing.assert_allclose(y_all[b], ref, rtol=1e-11, atol=1e-11)
    empty = lay.sparse_ffn(x, np.zeros(0, dtype=np.int32))
    assert np.all(empty == 0.0)
    bd = rng.standard_normal(d).astype(np.float32)
    lay_b = oracle.Layer(spec.act, n["w_up"], n["w_dT"], w_gate=n["w_gate"], s_up=n["s_up"], s_gate=n["s_gate"],
                         s_dT=n["s_dT"], b_up=n["b_up"], b_gate=n["b_gate"], b_down=bd)
    assert np.array_equal(lay_b.sparse_ffn(x, np.zeros(0, dtype=np.int32)), np.tile(bd.astype(np.float64), (8, 1)))


@pytest.mark.parametrize("name", ["tiny_relu_f32", "llama2_13b_swiglu_f16"])
def test_disjoint_additivity(name):
    spec, L, n, lay, x = _small_layer(name)
    perm = rng.permutation(lay.F)
    m1, m2 = np.sort(perm[:90]).astype(np.int32), np.sort(perm[90:200]).astype(np.int32)
    both = np.sort(np.concatenate([m1, m2])).astype(np.int32)
    np.testing.assert_allclose(lay.sparse_ffn(x, both), lay.sparse_ffn(x, m1) + lay.sparse_ffn(x, m2),
                               rtol=1e-12, atol=1e-12)


def test_relu_superset_of_firing_set_is_bit_exact_dense():
    spec, L, n, lay, x = _small_layer("opt30b_relu_f16")
    for b in range(3):
        z = n["w_up"].astype(np.float64) @ x[b].astype(np.float64) + n["b_up"].astype(np.float64)
        firing = np.flatnonzero(z > 0)
        extra = rng.choice(np.setdiff1d(np.arange(lay.F), firing), 20, replace=False)
        sup = np.sort(np.concatenate([firing, extra])).astype(np.int32)
        assert np.array_equal(lay.sparse_ffn(x[b:b + 1], sup), lay.dense_ffn(x[b:b + 1]))


def test_swiglu_masked_difference_identity():
    spec, L, n, lay, x = _small_layer("llama2_13b_swiglu_f16")
    keep = np.sort(rng.choice(lay.F, 100, replace=False)).astype(np.int32)
    drop = np.setdiff1d(np.arange(lay.F), keep)
    xb = x[0].astype(np.float64)
    g = n["w_gate"].astype(np.float64) @ xb + n["b_gate"].astype(np.float64)
    u = n["w_up"].astype(np.float64) @ xb
    expect = sum((g[i] / (1 + np.exp(-g[i])) * u[i]) * n["w_dT"][i].astype(np.float64) for i in drop)
    np.testing.assert_allclose(lay.dense_ffn(x[:1])[0] - lay.sparse_ffn(x[:1], keep)[0], expect, rtol=1e-9,
                               atol=1e-11)


def test_activations_match_formula():
    spec, L, n, lay, x = _small_layer("tiny_relu_f32")
    idx = np.array([0, 5, 77, 255], dtype=np.int32)
    a = lay.activations(x[:2], idx)
    z = n["w_up"][idx].astype(np.float64) @ x[:2].astype(np.float64).T + n["b_up"][idx, None]
    np.testing.assert_allclose(a, np.maximum(z, 0), rtol=1e-12, atol=1e-12)


def test_batch_union_equals_per_token_on_union():
    spec, L, n, lay, x = _small_layer("opt30b_relu_f16")
    logits = oracle.predict_logits(n["A"], n["Q"], n["c"], x[:4])
    U = oracle.compact(logits)
    yb = lay.sparse_ffn(x[:4], U)
    for b in range(4):
        assert np.array_equal(yb[b], lay.sparse_ffn(x[b:b + 1], U)[0])
    for b in range(4):
        assert set(oracle.compact(logits[b:b + 1])) <= set(U)


# ------------------------------------------------------------------ profile + hot-first order

def test_fire_counts_match_numpy():
    for name in ("tiny_relu_f32", "llama2_13b_swiglu_f16", "opt175b_relu_i4"):
        spec, L, n, lay, x = _small_layer(name)
        X = synth.make_tokens(spec, 20, seed=9, stream="profile", d=lay.d).numpy()
        cnt = lay.fire_counts(X)
        if spec.act == "relu":
            W = oracle.i4_dequant(n["w_up"], n["s_up"], lay.d) if lay.dt == oracle.I4G128 else n["w_up"].astype(
                np.float64)
            z = W @ X.astype(np.float64).T + n["b_up"].astype(np.float64)[:, None]
        else:
            z = n["w_gate"].astype(np.float64) @ X.astype(np.float64).T + n["b_gate"].astype(np.float64)[:, None]
        assert np.array_equal(cnt, (z > 0).sum(axis=1).astype(np.int32))
        for t in (-0.3, 0.25):
            assert np.array_equal(lay.fire_counts(X, t), (z > t).sum(axis=1).astype(np.int32))
        # the pre-activations themselves: numpy's fp64 product (a library routine), and the same
        # signs the counts come from
        za = lay.pre_activations(X)
        assert za.shape == (X.shape[0], lay.F)
        assert np.allclose(za, z.T, rtol=1e-12, atol=1e-12 * np.abs(z).max())
        assert np.array_equal((za > 0).sum(axis=0).astype(np.int32), cnt)


def test_compact_with_hot_prefix():
    # the hot prefix [0, n_hot) is kept whatever the logits; the rest follows the strict rule
    logits = rng.standard_normal((3, 400))
    logits[:, :50] = -5.0  # a hot neuron the predictor would drop is still kept
    for n_hot in (0, 1, 37, 64, 399, 400):
        got = oracle.compact(logits, 0.0, n_hot=n_hot)
        ref = sorted(set(range(n_hot)) | {i for i in range(400) if any(logits[b, i] > 0.0 for b in range(3))})
        assert np.array_equal(got, np.array(ref, dtype=np.int32)), n_hot
    assert np.array_equal(oracle.compact(logits, 0.0, n_hot=0), oracle.compact(logits, 0.0))
    assert np.array_equal(oracle.compact(np.full((1, 9), -1.0), 0.0, n_hot=9), np.arange(9))
    assert np.array_equal(oracle.compact(np.full((2, 9), -1.0), 0.0, n_hot=4), np.arange(4))
    # the tail equals the plain rule on the tail
    tail = oracle.compact(logits, 0.3, n_hot=120)
    assert np.array_equal(tail[tail >= 120], np.flatnonzero(logits.max(axis=0) > 0.3)[np.flatnonzero(logits.max(axis=0) > 0.3) >= 120])


def test_hot_first_perm_is_stable_descending_bijection():
    counts = rng.integers(0, 6, 3000).astype(np.int32)  # many ties
    perm = oracle.hot_first_perm(counts)
    assert np.array_equal(np.sort(perm), np.arange(3000))
    assert np.all(np.diff(counts[perm]) <= 0)
    ref = sorted(range(3000), key=lambda i: (-int(counts[i]), i))
    assert np.array_equal(perm, np.array(ref, dtype=np.int32))
    assert np.array_equal(oracle.hot_first_perm(np.zeros(5, np.int32)), np.arange(5))


def test_permutation_invariance():
    spec, L, n, lay, x = _small_layer("opt30b_relu_f16")
    X = synth.make_tokens(spec, 32, seed=2, stream="profile", d=lay.d).numpy()
    perm = oracle.hot_first_perm(lay.fire_counts(X))
    lg = oracle.predict_logits(n["A"], n["Q"], n["c"], x)
    lgp = oracle.predict_logits(n["A"], np.ascontiguousarray(n["Q"][perm]), np.ascontiguousarray(n["c"][perm]), x)
    assert np.array_equal(lgp, lg[:, perm])  # each logit depends only on its own row
    S = oracle.compact(lg[:1])
    Sp = oracle.compact(lgp[:1])
    inv = np.argsort(perm)
    assert np.array_equal(Sp, np.sort(inv[S]).astype(np.int32))
    lp = lay.permuted(perm)
    np.testing.assert_allclose(lp.sparse_ffn(x[:1], Sp), lay.sparse_ffn(x[:1], S), rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------------ layer norm + stack

def test_layernorm_closed_form_and_library():
    x = (rng.standard_normal((5, 300)) * 3 + 1.5).astype(np.float32)
    eps = 1e-5
    out = oracle.layernorm(x, eps)
    x64 = x.astype(np.float64)
    v = x64.var(axis=1)
    np.testing.assert_allclose(out.mean(axis=1), 0.0, atol=1e-13)
    np.testing.assert_allclose(out.var(axis=1), v / (v + eps), rtol=1e-12)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x64), (300,), eps=eps).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_stack_step_reduces_to_residual_identity_and_single_layer():
    spec = synth.CONFIGS["falcon40b_stack_f16"]
    d, F, r = 64, 128, 8
    layers = []
    for l in range(2):
        L = synth.make_layer(spec, seed=5, layer=l, d=d, F=F, r=r)
        n = L.numpy()
        layers.append((n["A"], n["Q"], n["c"], oracle.Layer("relu", n["w_up"], n["w_dT"], b_up=n["b_up"])))
    x0 = synth.make_residual(spec, 2, seed=5, d=d).numpy()
    # zero down-projection: the FFN adds nothing, the residual stream passes through unchanged
    A, Q, c, lay = layers[0]
    zero = oracle.Layer("relu", lay.w_up, np.zeros_like(lay.w_dT), b_up=lay.b_up)
    assert np.array_equal(oracle.stack_step([(A, Q, c, zero)], x0), x0)
    # one layer: x + FFN over the predicted set of fp16(LN(x)), written out with numpy
    h = torch.nn.functional.layer_norm(torch.from_numpy(x0.astype(np.float64)), (d,), eps=1e-5).numpy()
    h16 = h.astype(np.float16)
    x1 = oracle.stack_step(layers[:1], x0)
    lg = Q.astype(np.float64) @ (A.astype(np.float64) @ h16.astype(np.float64).T) + c.astype(np.float64)[:, None]
    keep = (lg > 0).any(axis=1).astype(np.float64)  # the batch shares the union of its tokens' sets
    for b in range(2):
        y = _np_relu_ffn(lay.w_up, lay.b_up, lay.w_dT, h16[b], keep)
        np.testing.assert_allclose(x1[b], (x0[b].astype(np.float64) + y).astype(np.float32), rtol=1e-6, atol=1e-6)
    x2 = oracle.stack_step(layers, x0)
    assert np.array_equal(x2, oracle.stack_step(layers[1:], x1))
