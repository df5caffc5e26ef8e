"""GPU parity of the HIP path against the CPU oracle on small ragged shapes (several tiles plus a
ragged tail in every dimension), every storage type and activation, batches 1..32, and the edge
lists (empty, all neurons, unordered, perfect predictor).  Calls go through the C ABI via the
Python binding; inputs come from the seeded generator."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import (BAND, check_counts, check_set, check_y, ffn_of, ln_bound, oracle_layer, pred_of, rel_inf,
                     spec_variant, tol_for)

pytestmark = pytest.mark.gpu

ps = pytest.importorskip("activation_sparse_ffn_psffn_amd")
DEV = "cuda"

# (label, base workload, overrides): d and F are not multiples of the kernels' tiles
CASES = [
    ("f32_relu", "tiny_relu_f32", dict(d=264, F=1000, r=40)),
    ("f16_relu", "opt30b_relu_f16", dict(d=1288, F=2000, r=136, density=0.05)),
    # more neurons than one interleave block of the one-token layer's logits kernel (256 chunks of 16),
    # with a ragged last block
    ("f16_relu_blocks", "opt30b_relu_f16", dict(d=776, F=5000, r=64, density=0.05)),
    ("f16_swiglu", "llama2_13b_swiglu_f16", dict(d=1032, F=1500, r=72)),
    ("i4_relu", "opt175b_relu_i4", dict(d=1152, F=1200, r=64, density=0.08)),
    ("i4_swiglu", "opt175b_relu_i4", dict(d=640, F=700, r=32, act="swiglu", density=0.4)),
    ("f32_swiglu", "tiny_relu_f32", dict(d=136, F=333, r=16, act="swiglu", density=0.3)),
    # rows wider than one pass of the small-batch kernels (fp16 > 8192, fp32 > 4096, 4-bit > 12288
    # elements) and more column slices than one pass of the down projection
    ("f16_relu_wide", "opt30b_relu_f16", dict(d=8200, F=600, r=24, density=0.1)),
    ("f32_relu_wide", "tiny_relu_f32", dict(d=4104, F=300, r=16)),
    ("i4_relu_wide", "opt175b_relu_i4", dict(d=12416, F=400, r=24, density=0.1)),
]

_cache = {}


def setup_case(label, seed=0):
    if label in _cache:
        return _cache[label]
    _, base, kw = next(c for c in CASES if c[0] == label)
    dims = {k: kw[k] for k in ("d", "F", "r")}
    spec = spec_variant(base, **{k: v for k, v in kw.items() if k not in dims})
    torch.cuda.synchronize()
    L = synth.make_layer(spec, seed=seed, device=DEV, **dims)
    n = L.numpy()
    X = synth.make_tokens(L.spec, 40, seed=seed, device=DEV)
    out = dict(spec=L.spec, L=L, n=n, X=X, Xn=X.cpu().numpy(), W=ffn_of(L, ps), P=pred_of(L, ps),
               orc=oracle_layer(n, L.spec.act))
    out["ws"] = ps.new_workspace(out["P"], out["W"], ps.MAX_BATCH)
    _cache[label] = out
    return out


def say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("label", [c[0] for c in CASES])
@pytest.mark.parametrize("B", [1, 2, 3, 4, 8, 32])
def test_predict_sets_and_logits(label, B):
    c = setup_case(label)
    say("predict", label, "B", B)
    x = c["X"][:B].contiguous()
    F = c["spec"].F
    logits = torch.empty(B, F, dtype=torch.float32, device=DEV)
    idx, count = ps.predict(c["P"], x, c["ws"], logits=logits)
    torch.cuda.synchronize()
    ref = oracle.predict_logits(c["n"]["A"], c["n"]["Q"], c["n"]["c"], c["Xn"][:B])
    st = check_set(idx, count, ref)
    dl = np.abs(logits.cpu().numpy().astype(np.float64) - ref).max()
    say("  count", st, "max|dlogit| %.2e" % dl)
    assert dl < 1e-5 * (1 + np.abs(ref).max())


# Ranks past what the batch predictor's whole-tile logits kernel holds in LDS: the kernel that keeps
# h in LDS (16 tokens up to 2552 ranks; 32 tokens up to 1272) and the one that reads h fragments
# from L2 (beyond those).  Predictor-only shapes with ragged d and F.
@pytest.mark.parametrize("r,B,kernel", [(1152, 20, "h in LDS, 32 tokens"), (1544, 8, "h in LDS, 16 tokens"),
                                        (1544, 24, "h from L2, 32 tokens"), (2560, 8, "h from L2, 16 tokens")])
def test_batch_predictor_large_ranks(r, B, kernel):
    say("batch predictor", "r", r, "B", B, kernel)
    spec = spec_variant("opt30b_relu_f16", density=0.05)
    L = synth.make_layer(spec, seed=3, device=DEV, d=520, F=700, r=r)
    n = L.numpy()
    P, W = pred_of(L, ps), ffn_of(L, ps)
    ws = ps.new_workspace(P, W, B)
    X = synth.make_tokens(L.spec, B, seed=11, device=DEV, d=520)
    logits = torch.empty(B, 700, device=DEV)
    idx, count = ps.predict(P, X, ws, logits=logits)
    torch.cuda.synchronize()
    ref = oracle.predict_logits(n["A"], n["Q"], n["c"], X.cpu().numpy())
    st = check_set(idx, count, ref)
    dl = np.abs(logits.cpu().numpy().astype(np.float64) - ref).max()
    assert dl < 1e-5 * (1 + np.abs(ref).max())
    idx2, cnt2, y = ps.layer(P, W, X, ws)
    torch.cuda.synchronize()
    m = int(count.item())
    assert int(cnt2.item()) == m and torch.equal(idx2[:m], idx[:m])
    if st["exact"]:
        check_y(y.cpu().numpy(), oracle_layer(n, "relu").sparse_ffn(X.cpu().numpy(), oracle.compact(ref)), 2e-3)
    say("  count", st, "max|dlogit| %.2e" % dl)


@pytest.mark.parametrize("label", [c[0] for c in CASES])
@pytest.mark.parametrize("B", [1, 2, 3, 4, 8, 32])
def test_sparse_ffn_on_oracle_list(label, B):
    c = setup_case(label)
    say("sparse_ffn", label, "B", B)
    x = c["X"][:B].contiguous()
    ref_logits = oracle.predict_logits(c["n"]["A"], c["n"]["Q"], c["n"]["c"], c["Xn"][:B])
    lst = oracle.compact(ref_logits)
    idx = torch.from_numpy(lst).to(DEV)
    count = torch.tensor([len(lst)], dtype=torch.int32, device=DEV)
    y = ps.sparse_ffn(c["W"], x, idx, count, c["ws"])
    torch.cuda.synchronize()
    y_ref = c["orc"].sparse_ffn(c["Xn"][:B], lst)
    e = check_y(y.cpu().numpy(), y_ref, tol_for(c["spec"].storage))
    say("  rows", len(lst), "rel err %.2e" % e)


@pytest.mark.parametrize("label", [c[0] for c in CASES])
@pytest.mark.parametrize("B", [1, 2, 8, 20])
def test_edge_lists(label, B):
    c = setup_case(label)
    say("edge lists", label, "B", B)
    F, d = c["spec"].F, c["spec"].d
    x = c["X"][:B].contiguous()
    xn = c["Xn"][:B]
    tol = tol_for(c["spec"].storage)
    # empty list: y = b_down exactly (and 0 without b_down)
    idx0 = torch.zeros(F, dtype=torch.int32, device=DEV)
    cnt0 = torch.zeros(1, dtype=torch.int32, device=DEV)
    y = ps.sparse_ffn(c["W"], x, idx0, cnt0, c["ws"])
    assert torch.count_nonzero(y).item() == 0
    bd = torch.randn(d, generator=torch.Generator().manual_seed(5)).to(DEV)
    Wb = ps.FFN(**{**c["W"].__dict__, "b_down": bd})
    y = ps.sparse_ffn(Wb, x, idx0, cnt0, c["ws"])
    assert torch.equal(y, bd.expand(B, d))
    # all neurons = dense FFN
    alln = np.arange(F, dtype=np.int32)
    y = ps.sparse_ffn(c["W"], x, torch.from_numpy(alln).to(DEV), torch.tensor([F], dtype=torch.int32, device=DEV),
                      c["ws"])
    check_y(y.cpu().numpy(), c["orc"].dense_ffn(xn), tol)
    # any order: a shuffled subset
    rng = np.random.default_rng(1)
    sub = rng.permutation(F)[: F // 3].astype(np.int32)
    y = ps.sparse_ffn(c["W"], x, torch.from_numpy(sub).to(DEV),
                      torch.tensor([len(sub)], dtype=torch.int32, device=DEV), c["ws"])
    check_y(y.cpu().numpy(), c["orc"].sparse_ffn(xn, sub), tol)
    # a single neuron, with b_down
    one = np.array([F - 1], dtype=np.int32)
    ob = oracle_layer(c["n"], c["spec"].act, b_down=bd.cpu().numpy())
    y = ps.sparse_ffn(Wb, x, torch.from_numpy(one).to(DEV), torch.tensor([1], dtype=torch.int32, device=DEV),
                      c["ws"])
    check_y(y.cpu().numpy(), ob.sparse_ffn(xn, one), tol)


@pytest.mark.parametrize("label", [c[0] for c in CASES])
@pytest.mark.parametrize("B", [1, 3, 8])
def test_extreme_thresholds(label, B):
    """No neuron above the threshold (empty list: y is zero, a residual is unchanged) and every
    neuron above it (the full list 0..F-1: the layer is the dense FFN), through both the predictor
    call and the one-call layer (which orders the list inside the FFN kernel)."""
    c = setup_case(label)
    say("extreme thresholds", label, "B", B)
    x = c["X"][:B].contiguous()
    F, d = c["spec"].F, c["spec"].d
    for thr in (1e30, -1e30):
        idx, cnt = ps.predict(c["P"], x, c["ws"], thr=thr)
        n_exp = 0 if thr > 0 else F
        assert int(cnt.item()) == n_exp
        if n_exp:
            assert torch.equal(idx.cpu(), torch.arange(F, dtype=torch.int32))
        idx2, cnt2, y = ps.layer(c["P"], c["W"], x, c["ws"], thr=thr)
        assert int(cnt2.item()) == n_exp
        if n_exp == 0:
            assert torch.count_nonzero(y).item() == 0
            base = torch.randn(B, d, generator=torch.Generator().manual_seed(3)).to(DEV)
            acc = base.clone()
            ps.layer(c["P"], c["W"], x, c["ws"], thr=thr, y=acc, accumulate=True)
            assert torch.equal(acc, base)
        else:
            assert torch.equal(idx2.cpu(), torch.arange(F, dtype=torch.int32))
            check_y(y.cpu().numpy(), c["orc"].dense_ffn(c["Xn"][:B]), tol_for(c["spec"].storage))


@pytest.mark.parametrize("label", ["f32_relu", "f16_relu", "i4_relu"])
def test_perfect_predictor_list_gives_dense(label):
    c = setup_case(label)
    say("perfect predictor", label)
    xn = c["Xn"][:1]
    dense = c["orc"].dense_ffn(xn)
    # the oracle's own firing set {z > 0}: neurons outside it contribute exactly 0 under ReLU
    z_cnt = c["orc"].fire_counts(xn)
    lst = np.flatnonzero(z_cnt > 0).astype(np.int32)
    assert np.array_equal(c["orc"].sparse_ffn(xn, lst), dense)
    y = ps.sparse_ffn(c["W"], c["X"][:1].contiguous(), torch.from_numpy(lst).to(DEV),
                      torch.tensor([len(lst)], dtype=torch.int32, device=DEV), c["ws"])
    check_y(y.cpu().numpy(), dense, tol_for(c["spec"].storage))


@pytest.mark.parametrize("label", ["f16_relu", "i4_relu", "f16_swiglu"])
@pytest.mark.parametrize("B", [1, 4, 12])
def test_accumulate_and_determinism(label, B):
    c = setup_case(label)
    say("accumulate/determinism", label, "B", B)
    x = c["X"][:B].contiguous()
    idx, count = ps.predict(c["P"], x, c["ws"])
    y1 = ps.sparse_ffn(c["W"], x, idx, count, c["ws"])
    idx2, count2 = ps.predict(c["P"], x, c["ws"])
    y2 = ps.sparse_ffn(c["W"], x, idx2, count2, c["ws"])
    torch.cuda.synchronize()
    n = int(count.item())
    assert int(count2.item()) == n and torch.equal(idx[:n], idx2[:n])
    assert torch.equal(y1, y2)
    base = torch.randn(B, c["spec"].d, generator=torch.Generator().manual_seed(2)).to(DEV)
    acc = base.clone()
    ps.sparse_ffn(c["W"], x, idx, count, c["ws"], y=acc, accumulate=True)
    assert torch.equal(acc, base + y1)


@pytest.mark.parametrize("B,F", [(1, 1), (1, 255), (3, 256), (5, 1000), (32, 4097)])
def test_compact_given_logits(B, F):
    say("compact", B, F)
    g = torch.Generator().manual_seed(B * 1000 + F)
    lg = torch.randn(B, F, generator=g, dtype=torch.float32) - 1.5
    lg[:, ::7] = 0.0  # exactly at the threshold: inactive
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=DEV)
    ps.workspace_init(ws)
    idx, count = ps.compact(lg.to(DEV), ws)
    ref = oracle.compact(lg.numpy().astype(np.float64), 0.0)
    n = int(count.item())
    assert n == len(ref)
    assert np.array_equal(idx[:n].cpu().numpy(), ref)
    idx, count = ps.compact(lg.to(DEV), ws, thr=0.5)
    ref = oracle.compact(lg.numpy().astype(np.float64), float(np.float32(0.5)))
    assert int(count.item()) == len(ref) and np.array_equal(idx[: len(ref)].cpu().numpy(), ref)


@pytest.mark.parametrize("label", [c[0] for c in CASES])
def test_profile_counts(label):
    c = setup_case(label)
    say("profile counts", label)
    T = 24
    Xp = synth.make_tokens(c["spec"], T, seed=4, stream="profile", device=DEV)
    Xpn = Xp.cpu().numpy()
    got = ps.profile_counts(c["W"], Xp).cpu().numpy()
    amb = check_counts(got, c["orc"], c["n"], Xpn)
    say("  neurons with a token inside the fp32 margin: %d of %d" % (amb, c["spec"].F))


@pytest.mark.parametrize("label", [c[0] for c in CASES])
def test_permute_hot_first(label):
    c = setup_case(label)
    say("permute", label)
    counts = synth.profile_like_counts(c["L"].p, 512, seed=3)
    perm_ref = oracle.hot_first_perm(counts)
    perm, W2, P2 = ps.permute_hot_first(torch.from_numpy(counts).to(DEV), c["W"], c["P"])
    torch.cuda.synchronize()
    assert np.array_equal(perm.cpu().numpy(), perm_ref)
    # the expected rows: the oracle's own reordering of the stored layer (new neuron k = old perm[k])
    op = c["orc"].permuted(perm_ref)
    for name in ("w_up", "w_gate", "w_dT", "s_up", "s_gate", "s_dT", "b_up", "b_gate"):
        a, b = getattr(W2, name), getattr(op, name)
        assert (a is None) == (b is None), name
        if a is not None:
            an = a.cpu().numpy()
            assert an.dtype == b.dtype and np.array_equal(an.view(np.uint8), b.view(np.uint8)), name
    Qp, cp = c["n"]["Q"][perm_ref], c["n"]["c"][perm_ref]
    assert np.array_equal(P2.Q.cpu().numpy().view(np.uint8), Qp.view(np.uint8))
    assert np.array_equal(P2.c.cpu().numpy().view(np.uint8), cp.view(np.uint8)) and P2.A is c["P"].A
    # each logit depends only on its own row: permuted logits are bit-identical
    x = c["X"][:3].contiguous()
    F = c["spec"].F
    l1 = torch.empty(3, F, device=DEV)
    l2 = torch.empty(3, F, device=DEV)
    ps.predict(c["P"], x, c["ws"], logits=l1)
    ps.predict(P2, x, c["ws"], logits=l2)
    assert torch.equal(l2, l1[:, perm.long()])


@pytest.mark.parametrize("B,d", [(1, 8192), (4, 1000), (32, 264), (3, 5), (32, 8192), (2, 12288)])
def test_layernorm_f16(B, d):
    say("layernorm", B, d)
    g = torch.Generator().manual_seed(B + d)
    x = (torch.randn(B, d, generator=g) * 3 + torch.randn(B, 1, generator=g) * 2).to(torch.float32)
    got = ps.layernorm_f16(x.to(DEV)).cpu().numpy().astype(np.float64)
    ref = oracle.layernorm(x.numpy(), 1e-5)
    # one fp16 ulp plus the near-zero slack of fp32 arithmetic (helpers.ln_bound).  A plain fp32
    # two-pass LayerNorm meets this bound; one with the variance taken about zero misses it on most
    # elements.
    assert np.all(np.abs(got - ref) <= ln_bound(x.numpy(), ref))


@pytest.mark.parametrize("label", [c[0] for c in CASES])
@pytest.mark.parametrize("B", [1, 2, 3, 4, 8, 20, 32])
def test_layer_call_equals_two_calls_and_oracle(label, B):
    c = setup_case(label)
    say("layer", label, "B", B)
    x = c["X"][:B].contiguous()
    F = c["spec"].F
    logits1 = torch.empty(B, F, device=DEV)
    idx1, cnt1 = ps.predict(c["P"], x, c["ws"], logits=logits1)
    y1 = ps.sparse_ffn(c["W"], x, idx1, cnt1, c["ws"])
    logits = torch.empty(B, F, device=DEV)
    idx2, cnt2, y2 = ps.layer(c["P"], c["W"], x, c["ws"], logits=logits)
    torch.cuda.synchronize()
    n = int(cnt1.item())
    # the same logit arithmetic in both paths: the same logits, the same list
    assert torch.equal(logits1, logits)
    assert int(cnt2.item()) == n and torch.equal(idx1[:n], idx2[:n])
    assert torch.equal(y1, y2)  # same kernels downstream of the list: bit-identical
    ref = oracle.predict_logits(c["n"]["A"], c["n"]["Q"], c["n"]["c"], c["Xn"][:B])
    st = check_set(idx2, cnt2, ref)
    if st["exact"]:
        check_y(y2.cpu().numpy(), c["orc"].sparse_ffn(c["Xn"][:B], oracle.compact(ref)), tol_for(c["spec"].storage))
    # accumulate into a residual, twice in a row on one workspace
    base = torch.randn(B, c["spec"].d, generator=torch.Generator().manual_seed(9)).to(DEV)
    acc = base.clone()
    ps.layer(c["P"], c["W"], x, c["ws"], y=acc, accumulate=True)
    ps.layer(c["P"], c["W"], x, c["ws"], y=acc, accumulate=True)
    assert torch.equal(acc, (base + y1) + y1)


@pytest.mark.parametrize("label,B,n_hot", [("f16_relu", 1, 0), ("f16_relu", 8, 0), ("i4_swiglu", 24, 0),
                                           ("f16_relu", 1, 101), ("f16_swiglu", 3, 700)])
def test_layer_graph_replay_matches_eager(label, B, n_hot):
    c = setup_case(label)
    say("graph replay", label, "B", B, "n_hot", n_hot)
    x = c["X"][:B].contiguous()
    idx, cnt, y = ps.layer(c["P"], c["W"], x, c["ws"], n_hot=n_hot)
    y_ref = y.clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            ps.layer(c["P"], c["W"], x, c["ws"], idx=idx, count=cnt, y=y, n_hot=n_hot)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(4):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), "replay %d differs" % rep
        ps.layer(c["P"], c["W"], x, c["ws"])  # eager work between replays on the same workspace
        torch.cuda.synchronize()


@pytest.mark.parametrize("label", [c[0] for c in CASES])
@pytest.mark.parametrize("B", [1, 2, 4, 8, 32])
def test_hot_prefix_predict_and_layer(label, B):
    # neurons [0, n_hot) are listed without prediction; the tail follows the predictor exactly as
    # in psffn_predict (same logits), and the layer call's y is the sparse FFN on that list
    c = setup_case(label)
    x = c["X"][:B].contiguous()
    F = c["spec"].F
    ref = oracle.predict_logits(c["n"]["A"], c["n"]["Q"], c["n"]["c"], c["Xn"][:B])
    logits0 = torch.empty(B, F, device=DEV)
    ps.predict(c["P"], x, c["ws"], logits=logits0)
    for n_hot in (1, 37, (F // 3) | 5, F - 3, F):
        say("hot prefix", label, "B", B, "n_hot", n_hot)
        logits = torch.empty(B, F, device=DEV)
        idx, cnt = ps.predict(c["P"], x, c["ws"], logits=logits, n_hot=n_hot)
        torch.cuda.synchronize()
        st = check_set(idx, cnt, ref, n_hot=n_hot)
        assert torch.equal(logits[:, n_hot:], logits0[:, n_hot:])
        n = int(cnt.item())
        assert n >= n_hot and torch.equal(idx[:n_hot].cpu(), torch.arange(n_hot, dtype=torch.int32))
        idx2, cnt2, y2 = ps.layer(c["P"], c["W"], x, c["ws"], n_hot=n_hot)
        y1 = ps.sparse_ffn(c["W"], x, idx, cnt, c["ws"])
        torch.cuda.synchronize()
        assert int(cnt2.item()) == n and torch.equal(idx2[:n], idx[:n])
        assert torch.equal(y1, y2)
        if st["exact"]:
            check_y(y2.cpu().numpy(), c["orc"].sparse_ffn(c["Xn"][:B], oracle.compact(ref, n_hot=n_hot)),
                    tol_for(c["spec"].storage))


@pytest.mark.parametrize("label", ["f16_relu", "f16_swiglu", "i4_relu", "i4_swiglu", "f16_relu_wide", "i4_relu_wide"])
@pytest.mark.parametrize("B", [1, 2, 3, 4, 8])
def test_layer_ln_equals_layernorm_then_layer(label, B):
    # the stack step in one call (LayerNorm folded into the small-batch layer's first kernel) gives
    # the bits of psffn_layernorm_f16 followed by psffn_layer accumulating into the residual
    c = setup_case(label)
    say("layer_ln", label, "B", B)
    d, F = c["spec"].d, c["spec"].F
    x0 = synth.make_residual(c["spec"], B, seed=5, device=DEV, d=d).contiguous()
    x1 = x0.clone()
    h1 = ps.layernorm_f16(x1)
    lg1 = torch.empty(B, F, device=DEV)
    idx1, cnt1, _ = ps.layer(c["P"], c["W"], h1, c["ws"], logits=lg1, y=x1, accumulate=True)
    x2 = x0.clone()
    lg2 = torch.empty(B, F, device=DEV)
    idx2, cnt2, h2 = ps.layer_ln(c["P"], c["W"], x2, c["ws"], logits=lg2)
    torch.cuda.synchronize()
    n = int(cnt1.item())
    assert torch.equal(h1, h2)
    assert torch.equal(lg1, lg2)
    assert int(cnt2.item()) == n and torch.equal(idx1[:n], idx2[:n])
    assert torch.equal(x1, x2)
    # and through a graph, replayed with eager work in between
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    x3 = x0.clone()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            ps.layer_ln(c["P"], c["W"], x3, c["ws"], h=h2, idx=idx2, count=cnt2, stream=st)
    torch.cuda.current_stream().wait_stream(st)
    for rep in range(3):
        x3.copy_(x0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(x3, x1), "replay %d differs" % rep
        ps.layer(c["P"], c["W"], h1, c["ws"])
        torch.cuda.synchronize()


def test_layer_ln_needs_an_fp16_predictor():
    c = setup_case("f32_relu")
    x = synth.make_residual(c["spec"], 1, seed=5, device=DEV, d=c["spec"].d).contiguous()
    with pytest.raises(ps.PsffnError):
        ps.layer_ln(c["P"], c["W"], x, c["ws"])


@pytest.mark.parametrize("F,B", [(262144, 1), (262144, 2), (98304, 8), (98305, 8)])
def test_largest_neuron_counts(F, B):
    # F = 262144: the most neurons the small-batch layer path orders (8192 mask words, 256 splits
    # of at most 1024 rows); F = 98304: the batch pipeline's limit; one more neuron: the generic
    # kernels take over.  Narrow rows keep the oracle fast.
    spec = spec_variant("opt30b_relu_f16", density=0.03)
    say("largest F", F, "B", B)
    L = synth.make_layer(spec, seed=2, device=DEV, d=64, F=F, r=16)
    n = L.numpy()
    W, P = ffn_of(L, ps), pred_of(L, ps)
    ws = ps.new_workspace(P, W, B)
    X = synth.make_tokens(L.spec, B, seed=3, device=DEV, d=64)
    Xn = X.cpu().numpy()
    logits = torch.empty(B, F, device=DEV)
    idx, cnt = ps.predict(P, X, ws, logits=logits)
    y1 = ps.sparse_ffn(W, X, idx, cnt, ws)
    idx2, cnt2, y2 = ps.layer(P, W, X, ws)
    torch.cuda.synchronize()
    ref = oracle.predict_logits(n["A"], n["Q"], n["c"], Xn)
    st = check_set(idx, cnt, ref)
    m = int(cnt.item())
    assert int(cnt2.item()) == m and torch.equal(idx2[:m], idx[:m]) and torch.equal(y1, y2)
    orc = oracle_layer(n, "relu")
    lst = oracle.compact(ref)
    y_o = ps.sparse_ffn(W, X, torch.from_numpy(lst).to(DEV), torch.tensor([len(lst)], dtype=torch.int32,
                                                                          device=DEV), ws)
    check_y(y_o.cpu().numpy(), orc.sparse_ffn(Xn, lst), tol_for("f16"))
    if st["exact"]:
        check_y(y1.cpu().numpy(), orc.sparse_ffn(Xn, lst), tol_for("f16"))


@pytest.mark.parametrize("d,B", [(32768, 1), (32776, 1), (16384, 4)])
def test_widest_rows(d, B):
    # B x d fp16 activations fill the small-batch kernels' 64 KB of LDS at d = 32768 (B = 1) and
    # d = 16384 (B = 4); one slice more and the generic kernels take over.  The stack step at these
    # widths takes the LayerNorm kernel (its in-kernel form covers d <= 16384).
    spec = spec_variant("opt30b_relu_f16", density=0.05)
    say("widest rows d", d, "B", B)
    L = synth.make_layer(spec, seed=4, device=DEV, d=d, F=600, r=24)
    n = L.numpy()
    W, P = ffn_of(L, ps), pred_of(L, ps)
    ws = ps.new_workspace(P, W, B)
    X = synth.make_tokens(L.spec, B, seed=5, device=DEV, d=d)
    Xn = X.cpu().numpy()
    idx, cnt = ps.predict(P, X, ws)
    y1 = ps.sparse_ffn(W, X, idx, cnt, ws)
    idx2, cnt2, y2 = ps.layer(P, W, X, ws)
    torch.cuda.synchronize()
    ref = oracle.predict_logits(n["A"], n["Q"], n["c"], Xn)
    st = check_set(idx, cnt, ref)
    m = int(cnt.item())
    assert int(cnt2.item()) == m and torch.equal(idx2[:m], idx[:m]) and torch.equal(y1, y2)
    lst = oracle.compact(ref)
    orc = oracle_layer(n, "relu")
    y_o = ps.sparse_ffn(W, X, torch.from_numpy(lst).to(DEV), torch.tensor([len(lst)], dtype=torch.int32,
                                                                          device=DEV), ws)
    check_y(y_o.cpu().numpy(), orc.sparse_ffn(Xn, lst), tol_for("f16"))
    if st["exact"]:
        check_y(y1.cpu().numpy(), orc.sparse_ffn(Xn, lst), tol_for("f16"))
    x0 = synth.make_residual(L.spec, B, seed=6, device=DEV, d=d)
    x1 = x0.clone()
    h1 = ps.layernorm_f16(x1)
    ps.layer(P, W, h1, ws, y=x1, accumulate=True)
    x2 = x0.clone()
    _, _, h2 = ps.layer_ln(P, W, x2, ws)
    torch.cuda.synchronize()
    assert torch.equal(h1, h2) and torch.equal(x1, x2)


@pytest.mark.parametrize("d,F", [(12288, 400), (16384, 400), (16512, 400), (128, 262144)])
def test_4bit_one_token_limits(d, F):
    # the one-token pipeline with 4-bit rows: h by k_h1 up to d = 12288 and by k_h above; 4-bit up
    # rows of at most 16384 elements (two 32-element slices per lane); one row more and the small-batch
    # kernels take over; F = 262144: the most neurons (8192 mask words) with one 512-column tile
    spec = spec_variant("opt175b_relu_i4", density=0.05)
    say("4-bit one token d", d, "F", F)
    L = synth.make_layer(spec, seed=7, device=DEV, d=d, F=F, r=24)
    n = L.numpy()
    W, P = ffn_of(L, ps), pred_of(L, ps)
    ws = ps.new_workspace(P, W, 1)
    X = synth.make_tokens(L.spec, 1, seed=8, device=DEV, d=d)
    Xn = X.cpu().numpy()
    idx, cnt = ps.predict(P, X, ws)
    y1 = ps.sparse_ffn(W, X, idx, cnt, ws)
    idx2, cnt2, y2 = ps.layer(P, W, X, ws)
    torch.cuda.synchronize()
    ref = oracle.predict_logits(n["A"], n["Q"], n["c"], Xn)
    st = check_set(idx, cnt, ref)
    m = int(cnt.item())
    assert int(cnt2.item()) == m and torch.equal(idx2[:m], idx[:m]) and torch.equal(y1, y2)
    lst = oracle.compact(ref)
    orc = oracle_layer(n, "relu")
    y_o = ps.sparse_ffn(W, X, torch.from_numpy(lst).to(DEV), torch.tensor([len(lst)], dtype=torch.int32,
                                                                          device=DEV), ws)
    check_y(y_o.cpu().numpy(), orc.sparse_ffn(Xn, lst), tol_for("i4"))
    if st["exact"]:
        check_y(y1.cpu().numpy(), orc.sparse_ffn(Xn, lst), tol_for("i4"))
