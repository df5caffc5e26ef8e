"""Calls with distinct workspaces are independent: several layer calls in flight at once on
different streams give, bit for bit, what each gives alone.  The calls are issued round-robin from
one host thread, and from one host thread per stream (the binding's ctypes calls release the
interpreter lock, so the library's host code runs concurrently too).  Cases cover the streamed
one-token pipeline (fp16 and 4-bit), the small-batch pipeline and the MFMA batch pipeline.  All
streams have the default priority."""
import threading

import pytest
import torch

from test_gpu_parity import DEV, setup_case

ps = pytest.importorskip("activation_sparse_ffn_psffn_amd")
pytestmark = pytest.mark.gpu

K = 3      # concurrent streams, one workspace each
REPS = 4   # calls per stream


def alone(c, xs, wss):
    ref = []
    for k in range(K):
        idx, cnt, y = ps.layer(c["P"], c["W"], xs[k], wss[k])
        torch.cuda.synchronize()
        n = int(cnt.item())
        ref.append((n, idx[:n].clone(), y.clone()))
    return ref


def check_same(ref, outs):
    for k in range(K):
        n, idx, y = ref[k]
        assert int(outs[k][1].item()) == n, "stream %d: count" % k
        assert torch.equal(outs[k][0][:n], idx), "stream %d: list" % k
        assert torch.equal(outs[k][2], y), "stream %d: y" % k


@pytest.mark.parametrize("label,B", [("f16_relu", 1), ("i4_relu", 1), ("f16_swiglu", 3), ("f16_relu", 8),
                                     ("i4_relu", 8)])
@pytest.mark.parametrize("threads", [False, True])
def test_distinct_workspaces_on_concurrent_streams(label, B, threads):
    c = setup_case(label)
    print("concurrent", label, "B", B, "threads", threads, flush=True)
    F, d = c["spec"].F, c["spec"].d
    xs = [c["X"][k * B:(k + 1) * B].contiguous() for k in range(K)]
    wss = [ps.new_workspace(c["P"], c["W"], B) for _ in range(K)]
    torch.cuda.synchronize()
    ref = alone(c, xs, wss)
    streams = [torch.cuda.Stream() for _ in range(K)]
    outs = [(torch.full((F,), -1, dtype=torch.int32, device=DEV), torch.zeros(1, dtype=torch.int32, device=DEV),
             torch.zeros(B, d, dtype=torch.float32, device=DEV)) for _ in range(K)]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())

    def run(k):
        for _ in range(REPS):
            ps.layer(c["P"], c["W"], xs[k], wss[k], idx=outs[k][0], count=outs[k][1], y=outs[k][2], stream=streams[k])

    if threads:
        ts = [threading.Thread(target=run, args=(k,)) for k in range(K)]
        for t in ts:
            t.start()
        for t in ts:
            t.join()
    else:
        for _ in range(REPS):
            for k in range(K):
                ps.layer(c["P"], c["W"], xs[k], wss[k], idx=outs[k][0], count=outs[k][1], y=outs[k][2],
                         stream=streams[k])
    torch.cuda.synchronize()
    check_same(ref, outs)
