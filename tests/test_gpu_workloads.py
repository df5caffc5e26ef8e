"""GPU parity at the full sizes of the five synthetic workloads, on sampled tokens the oracle can
compute one by one (32 tokens at batch 1 for each single-layer workload): active sets (bit-exact
outside the 1e-6 logit band; the tokens with a difference inside the band are counted), FFN outputs
on the oracle's own lists, and end-to-end predict -> sparse FFN on every sampled token whose GPU set
equals the oracle's set."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import check_counts, check_set, check_y, ffn_of, oracle_layer, pred_of, tol_for

pytestmark = pytest.mark.gpu

ps = pytest.importorskip("activation_sparse_ffn_psffn_amd")
DEV = "cuda"


def say(*a):
    print(*a, flush=True)


def run_tokens(L, n, X, B, ntok_y=None, hot_first_perm=None):
    """Predict + sparse FFN on the GPU for the batch X [B][d]; check against the oracle."""
    W, P = ffn_of(L, ps), pred_of(L, ps)
    ws = ps.new_workspace(P, W, B)
    F = L.spec.F
    logits = torch.empty(B, F, device=DEV)
    idx, count = ps.predict(P, X, ws, logits=logits)
    y = ps.sparse_ffn(W, X, idx, count, ws)
    torch.cuda.synchronize()
    Xn = X.cpu().numpy()
    orc = oracle_layer(n, L.spec.act)
    ref_logits = oracle.predict_logits(n["A"], n["Q"], n["c"], Xn)
    st = check_set(idx, count, ref_logits)
    lst = oracle.compact(ref_logits)
    tb = B if ntok_y is None else ntok_y
    tol = tol_for(L.spec.storage)
    y_ref = orc.sparse_ffn(Xn[:tb], lst)
    # the sparse FFN on the oracle's list
    y_o = ps.sparse_ffn(W, X, torch.from_numpy(lst).to(DEV), torch.tensor([len(lst)], dtype=torch.int32,
                                                                          device=DEV), ws)
    e1 = check_y(y_o.cpu().numpy()[:tb], y_ref, tol)
    e2 = None
    if st["exact"]:
        e2 = check_y(y.cpu().numpy()[:tb], y_ref, tol)
    # the one-call layer the benchmark times: the same list, count and output, bit for bit
    logits2 = torch.empty(B, F, device=DEV)
    idx2, count2, y2 = ps.layer(P, W, X, ws, logits=logits2)
    torch.cuda.synchronize()
    n_gpu = int(count.item())
    assert torch.equal(logits2, logits)
    assert int(count2.item()) == n_gpu and torch.equal(idx2[:n_gpu], idx[:n_gpu])
    assert torch.equal(y2, y)
    say("  B=%d count=%d ref=%d in-band diffs=%d err(list)=%.2e err(end-to-end)=%s" % (
        B, st["count"], st["ref_count"], st["in_band_diff"], e1, "skipped" if e2 is None else "%.2e" % e2))
    return st


def tokens_b1(L, n, X, ntok):
    """run_tokens at batch 1 on the first ntok tokens; returns how many had the oracle's exact set
    (the others differ only inside the logit band)."""
    sts = [run_tokens(L, n, X[t:t + 1].contiguous(), 1) for t in range(ntok)]
    exact = sum(st["exact"] for st in sts)
    say("  %d tokens at batch 1: %d with the oracle's exact set, %d with differences inside the band "
        "(%d neurons in all)" % (ntok, exact, ntok - exact, sum(st["in_band_diff"] for st in sts)))
    return exact


def test_tiny_relu_f32_all_tokens():
    spec = synth.CONFIGS["tiny_relu_f32"]
    L = synth.make_layer(spec, seed=0, device=DEV)
    n = L.numpy()
    X = synth.make_tokens(spec, spec.tokens, seed=0, device=DEV)
    exact = 0
    for t in range(spec.tokens):
        exact += run_tokens(L, n, X[t:t + 1].contiguous(), 1)["exact"]
    assert exact >= spec.tokens - 2


def test_opt30b_relu_f16_hot_first():
    spec = synth.CONFIGS["opt30b_relu_f16"]
    say("generate", spec.name)
    L0 = synth.make_layer(spec, seed=0, device=DEV)
    counts = synth.profile_like_counts(L0.p, spec.profile_tokens, seed=0)
    perm_ref = oracle.hot_first_perm(counts)
    perm, W2, P2 = ps.permute_hot_first(torch.from_numpy(counts).to(DEV), ffn_of(L0, ps), pred_of(L0, ps))
    torch.cuda.synchronize()
    assert np.array_equal(perm.cpu().numpy(), perm_ref)
    L = L0.permuted(torch.from_numpy(perm_ref.astype(np.int64)))
    assert torch.equal(W2.w_up, L.w_up) and torch.equal(W2.w_dT, L.w_dT) and torch.equal(P2.Q, L.Q)
    del W2, P2
    n = L.numpy()
    X = synth.make_tokens(spec, 40, seed=0, device=DEV)
    exact = tokens_b1(L, n, X, 32)
    assert exact >= 28
    # two tokens (small-batch kernels) and four (batch pipeline)
    run_tokens(L, n, X[32:34].contiguous(), 2, ntok_y=1)
    run_tokens(L, n, X[34:38].contiguous(), 4, ntok_y=1)
    # the offline profile at full size, one token, within the fp32-accumulation bracket
    Xp = synth.make_tokens(spec, 1, seed=0, stream="profile", device=DEV)
    got = ps.profile_counts(ffn_of(L, ps), Xp).cpu().numpy()
    amb = check_counts(got, oracle_layer(n, "relu"), n, Xp.cpu().numpy())
    say("  profile: neurons with the token inside the fp32 margin: %d of %d" % (amb, spec.F))


def test_llama2_13b_swiglu_f16():
    spec = synth.CONFIGS["llama2_13b_swiglu_f16"]
    say("generate", spec.name)
    L = synth.make_layer(spec, seed=0, device=DEV)
    n = L.numpy()
    X = synth.make_tokens(spec, 35, seed=0, device=DEV)
    exact = tokens_b1(L, n, X, 32)
    assert exact >= 28
    # three tokens: the batch predictor with the small-batch FFN (one call ordering the list)
    run_tokens(L, n, X[32:35].contiguous(), 3, ntok_y=1)


def test_opt175b_relu_i4_batch1_2_and_8():
    spec = synth.CONFIGS["opt175b_relu_i4"]
    say("generate", spec.name)
    L = synth.make_layer(spec, seed=0, device=DEV)
    n = L.numpy()
    X = synth.make_tokens(spec, 40, seed=0, device=DEV)
    exact = tokens_b1(L, n, X, 32)
    run_tokens(L, n, X[32:40].contiguous(), 8, ntok_y=2)
    run_tokens(L, n, X[32:34].contiguous(), 2, ntok_y=1)  # 4-bit weights take the batch pipeline from 2 tokens
    assert exact >= 28


@pytest.mark.parametrize("layer,B", [(0, 1), (11, 2), (47, 4), (23, 32)])
def test_falcon40b_stack_layers(layer, B):
    spec = synth.CONFIGS["falcon40b_stack_f16"]
    say("generate", spec.name, "layer", layer, "density %.4f" % synth.layer_density(spec, 0, layer))
    L = synth.make_layer(spec, seed=0, layer=layer, device=DEV)
    n = L.numpy()
    X = synth.make_tokens(spec, B, seed=layer, device=DEV)
    run_tokens(L, n, X, B, ntok_y=min(B, 2))
    # the stack step the benchmark times (LayerNorm folded into the layer call where the small-batch
    # pipeline runs) against the LayerNorm kernel followed by the layer call: the same bits
    W, P = ffn_of(L, ps), pred_of(L, ps)
    ws = ps.new_workspace(P, W, B)
    x0 = synth.make_residual(spec, B, seed=layer, device=DEV)
    x1 = x0.clone()
    h1 = ps.layernorm_f16(x1)
    idx1, cnt1, _ = ps.layer(P, W, h1, ws, y=x1, accumulate=True)
    x2 = x0.clone()
    idx2, cnt2, h2 = ps.layer_ln(P, W, x2, ws)
    torch.cuda.synchronize()
    m = int(cnt1.item())
    assert torch.equal(h1, h2) and torch.equal(x1, x2)
    assert int(cnt2.item()) == m and torch.equal(idx1[:m], idx2[:m])
