"""Checks of the synthetic-input construction: the Zipf firing law, and that the biases make a
neuron (and its predictor logit) fire with the intended probability for x ~ N(0, I)."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth


@pytest.mark.parametrize("F,s,rho", [(1024, 1.1, 0.10), (28672, 1.1, 0.03), (13824, 0.8, 0.57), (49152, 1.1, 0.03),
                                     (32768, 1.0, 0.02), (32768, 1.0, 0.10)])
def test_zipf_probs_mean_clip_and_order(F, s, rho):
    p = synth.zipf_firing_probs(F, s, rho)
    assert abs(p.mean() - rho) < 1e-12
    assert p.max() <= synth.P_MAX and p.min() > 0
    assert np.all(np.diff(p) <= 0)  # rank order
    k = np.arange(1, F + 1, dtype=np.float64)
    free = p < synth.P_MAX
    ratio = p[free] / k[free] ** (-s)  # unclipped part is one constant times k^-s
    assert np.allclose(ratio, ratio[0], rtol=1e-12)


def test_expected_active_counts_of_the_workloads():
    # E|A| = sum of p = F * density, the expected number of active neurons per token
    for name, want in [("opt30b_relu_f16", 860.16), ("llama2_13b_swiglu_f16", 7879.68), ("opt175b_relu_i4", 1474.56)]:
        spec = synth.CONFIGS[name]
        assert abs(synth.neuron_probs(spec, seed=0).sum() - want) < 1e-6


def test_stack_layer_densities_in_range_and_seeded():
    spec = synth.CONFIGS["falcon40b_stack_f16"]
    ds = [synth.layer_density(spec, 0, l) for l in range(48)]
    assert all(0.02 <= v <= 0.10 for v in ds) and len(set(ds)) == 48
    assert ds == [synth.layer_density(spec, 0, l) for l in range(48)]


def test_firing_rates_match_probabilities():
    spec = synth.CONFIGS["tiny_relu_f32"]
    L = synth.make_layer(spec, seed=11)
    n = L.numpy()
    X = synth.make_tokens(spec, 4000, seed=11).numpy().astype(np.float64)
    z = n["w_up"].astype(np.float64) @ X.T + n["b_up"].astype(np.float64)[:, None]
    l = (n["Q"].astype(np.float64) @ (n["A"].astype(np.float64) @ X.T)) + n["c"].astype(np.float64)[:, None]
    p = L.p
    sd = np.sqrt(p * (1 - p) / X.shape[0])
    for emp in ((z > 0).mean(axis=1), (l > 0).mean(axis=1)):
        zscore = (emp - p) / sd
        assert np.abs(zscore).max() < 5.5
        assert abs(zscore.mean()) < 0.2  # no systematic bias over 1024 neurons
    # predicted count per token ~ sum p
    cnt = (l > 0).sum(axis=0)
    assert abs(cnt.mean() - p.sum()) < 4 * math.sqrt((p * (1 - p)).sum() / X.shape[0]) + 1e-9


def test_generation_is_seeded_and_order_independent():
    spec = synth.CONFIGS["opt175b_relu_i4"]
    a = synth.make_layer(spec, seed=3, d=256, F=64, r=8)
    b = synth.make_layer(spec, seed=3, d=256, F=64, r=8)
    c = synth.make_layer(spec, seed=4, d=256, F=64, r=8)
    assert torch.equal(a.w_up, b.w_up) and torch.equal(a.s_dT, b.s_dT) and torch.equal(a.c, b.c)
    assert not torch.equal(a.w_up, c.w_up)
    assert a.w_up.dtype == torch.uint8 and a.w_up.shape == (64, 128) and a.s_up.shape == (64, 2)
    assert a.A.dtype == torch.float16 and a.Q.shape == (64, 8)
