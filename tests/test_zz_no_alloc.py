"""psffn_layer_noalloc (the layer call on the library's static per-GPU scratch, no workspace
argument) against psffn_layer with a caller workspace, on the same seeded inputs: two calls in a
row on one GPU, the second on a smaller layer and batch, so the second call runs on scratch the
first one left behind.  Active lists must match exactly, outputs within the storage's tolerance."""
import numpy as np
import pytest
import torch

import synth
from helpers import check_y, ffn_of, pred_of, spec_variant, tol_for

pytestmark = pytest.mark.gpu

ps = pytest.importorskip("activation_sparse_ffn_psffn_amd")
DEV = "cuda"

# (base workload, dims, other overrides, batch): the second call is smaller in every dimension
CALLS = [
    ("opt30b_relu_f16", dict(d=1288, F=2000, r=136), dict(density=0.05), 4),
    ("opt30b_relu_f16", dict(d=520, F=700, r=40), dict(density=0.05), 1),
]


def _run(base, dims, kw, B, seed):
    spec = spec_variant(base, **kw)
    L = synth.make_layer(spec, seed=seed, device=DEV, **dims)
    x = synth.make_tokens(L.spec, B, seed=seed, device=DEV)
    P, W = pred_of(L, ps), ffn_of(L, ps)
    print("noalloc call", base, dims, "B", B, flush=True)
    idx_n, cnt_n, y_n = ps.layer_noalloc(P, W, x)
    torch.cuda.synchronize()
    ws = ps.new_workspace(P, W, B)
    idx_w, cnt_w, y_w = ps.layer(P, W, x, ws)
    torch.cuda.synchronize()
    n = int(cnt_w.item())
    assert int(cnt_n.item()) == n
    assert np.array_equal(idx_n[:n].cpu().numpy(), idx_w[:n].cpu().numpy())
    e = check_y(y_n.cpu().numpy(), y_w.cpu().numpy(), tol_for(L.spec.storage))
    print("  listed", n, "max rel diff %.2e" % e, flush=True)
    return n


def test_noalloc_two_calls_second_smaller():
    counts = [_run(base, dims, kw, B, seed=7 + k) for k, (base, dims, kw, B) in enumerate(CALLS)]
    assert all(c > 0 for c in counts)
