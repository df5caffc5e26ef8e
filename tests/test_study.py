"""The predictor-accuracy study: the aligned predictor input (CPU pins) and the study's statistics
from the HIP path against the same statistics from the oracle (GPU)."""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import BAND, oracle_layer

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402  (set_stats, cosine: host arithmetic on kernel outputs)


def _small(act="relu", storage="f16"):
    base = "llama2_13b_swiglu_f16" if act == "swiglu" else "opt30b_relu_f16"
    spec = synth.CONFIGS[base]
    if storage == "f32":
        from dataclasses import replace
        spec = replace(spec, storage="f32")
    return synth.make_layer(spec, seed=3, d=256, F=768, r=32)


@pytest.mark.parametrize("act", ["relu", "swiglu"])
def test_aligned_predictor_is_a_near_optimal_low_rank_factorisation(act):
    L = _small(act, "f32")
    Wd = (L.w_gate if act == "swiglu" else L.w_up).double()
    sv = torch.linalg.svdvals(Wd)
    for r in (8, 32, 128):
        A, Q, c = synth.make_aligned_predictor(L, r)
        assert A.shape == (r, 256) and Q.shape == (768, r) and c.shape == (768,)
        err = torch.linalg.norm(Q.double() @ A.double() - Wd) / torch.linalg.norm(Wd)
        best = torch.sqrt((sv[r:] ** 2).sum() / (sv ** 2).sum())  # Eckart-Young
        assert best <= err <= best * 1.05 + 1e-6, (r, float(err), float(best))  # randomized: within 5%
    # at full rank the predictor reproduces the pre-activations: logits = W x + b
    A, Q, c = synth.make_aligned_predictor(L, 256)
    x = synth.make_tokens(L.spec, 4, seed=1, d=256).numpy()
    lg = oracle.predict_logits(A.numpy(), Q.numpy(), c.numpy(), x)
    b = (L.b_gate if act == "swiglu" else L.b_up).double().numpy()
    z = x.astype(np.float64) @ Wd.numpy().T + b
    assert np.abs(lg - z).max() < 1e-4 * np.abs(z).max()


def test_set_stats_and_cosine():
    fired = np.zeros(10, bool)
    fired[[1, 2, 3, 7]] = True
    assert bench.set_stats(np.array([1, 2, 9]), fired) == (0.5, 2 / 3)
    assert bench.set_stats(np.array([], int), fired) == (0.0, 1.0)
    assert bench.set_stats(np.array([4]), np.zeros(10, bool)) == (1.0, 0.0)
    assert bench.cosine([1, 0], [2, 0]) == 1.0 and abs(bench.cosine([1, 0], [0, 3])) == 0.0
    assert bench.cosine([0, 0], [0, 0]) == 1.0


@pytest.mark.gpu
@pytest.mark.parametrize("act", ["relu", "swiglu"])
def test_study_statistics_match_the_oracle(act):
    ps = pytest.importorskip("activation_sparse_ffn_psffn_amd")
    dev = "cuda"
    L = _small(act)
    Ld = synth.make_layer(L.spec, seed=3, device=dev, d=256, F=768, r=32)
    n = Ld.numpy()
    W = ps.FFN(act, Ld.w_up, Ld.w_dT, w_gate=Ld.w_gate, b_up=Ld.b_up, b_gate=Ld.b_gate)
    orc = oracle_layer(n, act)
    X = synth.make_tokens(L.spec, 6, seed=2, device=dev, d=256)
    Xn = X.cpu().numpy()
    F = 768
    all_idx = torch.arange(F, dtype=torch.int32, device=dev)
    all_cnt = torch.tensor([F], dtype=torch.int32, device=dev)
    for r in (16, 64):
        A, Q, c = synth.make_aligned_predictor(Ld, r)
        P = ps.Predictor(A, Q, c)
        ws = ps.new_workspace(P, W, 1)
        ref_lg = oracle.predict_logits(A.cpu().numpy(), Q.cpu().numpy(), c.cpu().numpy(), Xn)
        for t in range(6):
            print("study stats", act, "rank", r, "token", t, flush=True)
            x = X[t:t + 1]
            fired = ps.profile_counts(W, x).cpu().numpy() > 0
            assert np.array_equal(fired, orc.fire_counts(Xn[t:t + 1]) > 0)
            idx, cnt, y = ps.layer(P, W, x, ws)
            dense = ps.sparse_ffn(W, x, all_idx, all_cnt, ws).cpu().numpy()
            got = idx[:int(cnt.item())].cpu().numpy()
            ref = oracle.compact(ref_lg[t:t + 1])
            if np.abs(ref_lg[t]).min() < BAND:
                continue  # a neuron in the band: the set may differ legitimately
            assert np.array_equal(got, ref)
            assert bench.set_stats(got, fired) == bench.set_stats(ref, fired)
            y_ref = orc.sparse_ffn(Xn[t:t + 1], ref)
            d_ref = orc.dense_ffn(Xn[t:t + 1])
            assert abs(bench.cosine(y.cpu().numpy(), dense) - bench.cosine(y_ref, d_ref)) < 1e-5
