"""Host-side contract of the C ABI (no GPU needed, no kernel is launched): the library loads,
exports every function include/psffn.h declares, and rejects invalid arguments with the
documented status before enqueuing anything.

Every call below carries at least one invalid argument, so validation returns before any HIP
call: the fake addresses are never handed to a kernel, on any host."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "psffn.h")

ps = pytest.importorskip("activation_sparse_ffn_psffn_amd")
lib = ps._lib

OK, INVALID, UNSUPPORTED, WORKSPACE = ps.PSFFN_OK, ps.PSFFN_E_INVALID_ARG, ps.PSFFN_E_UNSUPPORTED, ps.PSFFN_E_WORKSPACE

# fake, suitably aligned device addresses: validation never dereferences them
A16 = 0x7F0000000000
ADDR = iter(range(A16, A16 + (1 << 40), 1 << 28))


def fake():
    return next(ADDR)


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(psffn_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_function_is_exported():
    names = declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), n  # ctypes resolves the symbol or raises AttributeError
    assert set(names) == set(ps.EXPORTED)


def test_status_strings():
    for s in range(5):
        assert ps.status_str(s)
    assert ps.status_str(99) == "unknown status"


def pred(d=256, F=1024, r=32, dt=ps.PSFFN_F16, A=None, Q=None, c=None):
    return ps._Predictor(d, F, r, dt, fake() if A is None else A, fake() if Q is None else Q,
                         fake() if c is None else c)


def ffn(d=256, F=1024, dt=ps.PSFFN_F16, act=ps.PSFFN_RELU, **kw):
    f = dict(w_up=fake(), w_gate=None, w_dT=fake(), s_up=None, s_gate=None, s_dT=None, b_up=fake(), b_gate=None,
             b_down=None)
    if dt == ps.PSFFN_I4G128:
        f.update(s_up=fake(), s_dT=fake())
    if act == ps.PSFFN_SWIGLU:
        f.update(w_gate=fake(), b_gate=fake())
        if dt == ps.PSFFN_I4G128:
            f.update(s_gate=fake())
    f.update(kw)
    return ps._FFN(d, F, dt, act, f["w_up"], f["w_gate"], f["w_dT"], f["s_up"], f["s_gate"], f["s_dT"], f["b_up"],
                   f["b_gate"], f["b_down"])


B = ctypes.byref


def test_workspace_bytes():
    P, W = pred(), ffn()
    n1 = lib.psffn_workspace_bytes(B(P), None, 1)
    n2 = lib.psffn_workspace_bytes(B(P), B(W), 1)
    n8 = lib.psffn_workspace_bytes(B(P), B(W), 8)
    assert 0 < n1 <= n2 < n8
    assert lib.psffn_workspace_bytes(None, None, 1) == 0
    assert lib.psffn_workspace_bytes(B(P), B(W), 0) == 0
    assert lib.psffn_workspace_bytes(B(P), B(W), ps.MAX_BATCH + 1) == 0
    assert lib.psffn_workspace_bytes(B(pred(r=30)), None, 1) == 0


def call_predict(P, x=None, Bn=1, thr=0.0, idx=None, count=None, logits=None, ws=None, nbytes=1 << 30):
    return lib.psffn_predict(B(P), fake() if x is None else x, Bn, thr, fake() if idx is None else idx,
                             fake() if count is None else count, logits, fake() if ws is None else ws, nbytes, None)


def test_predict_rejects_bad_arguments():
    assert lib.psffn_predict(None, fake(), 1, 0.0, fake(), fake(), None, fake(), 1 << 30, None) == INVALID
    assert call_predict(pred(d=0)) == INVALID
    assert call_predict(pred(F=-1)) == INVALID
    assert call_predict(pred(dt=ps.PSFFN_I4G128)) == UNSUPPORTED  # 4-bit predictors are not provided
    assert call_predict(pred(dt=7)) == UNSUPPORTED
    assert call_predict(pred(d=260)) == UNSUPPORTED  # d % 8
    assert call_predict(pred(r=36)) == UNSUPPORTED  # r % 8
    assert call_predict(pred(A=A16 + 4)) == INVALID  # misaligned
    assert call_predict(pred(), Bn=0) == INVALID
    assert call_predict(pred(), Bn=33) == INVALID
    assert call_predict(pred(), x=A16 + 2) == INVALID
    assert call_predict(pred(), thr=float("nan")) == INVALID
    assert lib.psffn_predict(B(pred()), fake(), 1, 0.0, None, fake(), None, fake(), 1 << 30, None) == INVALID
    assert lib.psffn_predict(B(pred()), fake(), 1, 0.0, fake(), None, None, fake(), 1 << 30, None) == INVALID
    assert call_predict(pred(), ws=A16 + 128) == WORKSPACE  # 256-byte alignment
    need = lib.psffn_workspace_bytes(B(pred()), None, 1)
    assert call_predict(pred(), nbytes=need - 1) == WORKSPACE
    assert lib.psffn_predict(B(pred()), fake(), 1, 0.0, fake(), fake(), None, None, 1 << 30, None) == WORKSPACE


def test_compact_rejects_bad_arguments():
    assert lib.psffn_compact(None, 1, 10, 0.0, fake(), fake(), fake(), 1 << 20, None) == INVALID
    assert lib.psffn_compact(fake(), 1, 0, 0.0, fake(), fake(), fake(), 1 << 20, None) == INVALID
    assert lib.psffn_compact(fake(), 40, 10, 0.0, fake(), fake(), fake(), 1 << 20, None) == INVALID
    assert lib.psffn_compact(fake(), 1, 10, 0.0, fake(), fake(), fake(), 100, None) == WORKSPACE


def call_ffn(W, x=None, Bn=1, y=None, ws=None, nbytes=1 << 34):
    return lib.psffn_sparse_ffn(B(W), fake() if x is None else x, Bn, fake(), fake(), fake() if y is None else y, 0,
                                fake() if ws is None else ws, nbytes, None)


def test_sparse_ffn_rejects_bad_arguments():
    assert lib.psffn_sparse_ffn(None, fake(), 1, fake(), fake(), fake(), 0, fake(), 1 << 30, None) == INVALID
    assert call_ffn(ffn(act=5)) == UNSUPPORTED
    assert call_ffn(ffn(dt=ps.PSFFN_I4G128, d=192)) == UNSUPPORTED  # 4-bit needs d % 128
    assert call_ffn(ffn(d=100)) == UNSUPPORTED
    assert call_ffn(ffn(act=ps.PSFFN_SWIGLU, w_gate=None)) == INVALID
    assert call_ffn(ffn(dt=ps.PSFFN_I4G128, s_up=None)) == INVALID
    assert call_ffn(ffn(dt=ps.PSFFN_I4G128, act=ps.PSFFN_SWIGLU, s_gate=None)) == INVALID
    assert call_ffn(ffn(w_dT=A16 + 8)) == INVALID
    assert call_ffn(ffn(b_up=A16 + 2)) == INVALID
    assert call_ffn(ffn(), Bn=0) == INVALID
    assert lib.psffn_sparse_ffn(B(ffn()), fake(), 1, fake(), fake(), None, 0, fake(), 1 << 30, None) == INVALID
    need = lib.psffn_workspace_bytes(None, B(ffn()), 4)
    assert call_ffn(ffn(), Bn=4, nbytes=need - 256) == WORKSPACE


def test_profile_and_layernorm_reject_bad_arguments():
    assert lib.psffn_profile_counts(B(ffn()), fake(), 0, fake(), None) == INVALID
    assert lib.psffn_profile_counts(B(ffn()), None, 4, fake(), None) == INVALID
    assert lib.psffn_profile_counts(B(ffn(dt=9)), fake(), 4, fake(), None) == UNSUPPORTED
    assert lib.psffn_layernorm_f16(fake(), 0, 8, 1e-5, fake(), None) == INVALID
    assert lib.psffn_layernorm_f16(fake(), 1, 8, -1.0, fake(), None) == INVALID
    assert lib.psffn_layernorm_f16(None, 1, 8, 1e-5, fake(), None) == INVALID


def test_permute_rejects_bad_arguments():
    W, W2 = ffn(), ffn()
    assert lib.psffn_permute_hot_first(None, 1024, fake(), None, None, None, None, None) == INVALID
    assert lib.psffn_permute_hot_first(fake(), 0, fake(), None, None, None, None, None) == INVALID
    assert lib.psffn_permute_hot_first(fake(), 1024, fake(), B(W), None, None, None, None) == INVALID
    assert lib.psffn_permute_hot_first(fake(), 512, fake(), B(W), B(W2), None, None, None) == INVALID
    # destination overlapping the source
    W3 = ffn(w_up=W.w_up + 64)
    assert lib.psffn_permute_hot_first(fake(), 1024, fake(), B(W), B(W3), None, None, None) == INVALID
    # source has b_up but destination lacks it
    W4 = ffn(b_up=None)
    assert lib.psffn_permute_hot_first(fake(), 1024, fake(), B(W), B(W4), None, None, None) == INVALID
    P1, P2 = pred(), pred(r=64)
    assert lib.psffn_permute_hot_first(fake(), 1024, fake(), None, None, B(P1), B(P2), None) == INVALID


def test_workspace_init_rejects_bad_arguments():
    assert lib.psffn_workspace_init(None, 1024, None) == WORKSPACE
    assert lib.psffn_workspace_init(A16 + 16, 1024, None) == WORKSPACE
    assert lib.psffn_workspace_init(A16, 1000, None) == WORKSPACE


def test_hot_prefix_calls_reject_bad_prefix():
    P, W = pred(F=1024), ffn(F=1024)
    for n_hot in (-1, 1025):
        assert lib.psffn_predict_hot(B(P), n_hot, fake(), 1, 0.0, fake(), fake(), None, fake(), 1 << 30,
                                     None) == INVALID
        assert lib.psffn_layer_hot(B(P), B(W), n_hot, fake(), 1, 0.0, fake(), fake(), None, fake(), 0, fake(),
                                   1 << 34, None) == INVALID
    # the remaining checks are those of psffn_predict / psffn_layer
    assert lib.psffn_predict_hot(B(pred(d=260)), 4, fake(), 1, 0.0, fake(), fake(), None, fake(), 1 << 30,
                                 None) == UNSUPPORTED
    assert lib.psffn_layer_hot(B(P), B(W), 4, fake(), 0, 0.0, fake(), fake(), None, fake(), 0, fake(), 1 << 34,
                               None) == INVALID


def test_layer_ln_rejects_bad_arguments():
    P, W = pred(F=1024), ffn(F=1024)
    x, h = fake(), fake()
    call = lambda P=P, x=x, h=h, eps=1e-5, Bn=1: lib.psffn_layer_ln(B(P), B(W), x, eps, h, Bn, 0.0, fake(), fake(),
                                                                     None, fake(), 1 << 34, None)
    assert call(P=pred(F=1024, dt=ps.PSFFN_F32)) == UNSUPPORTED
    assert call(h=x) == INVALID  # the LayerNorm output overlaps the residual
    assert call(h=x + 256 * 4 - 16) == INVALID  # partial overlap (B = 1, d = 256: the residual is 1 KB)
    assert call(h=A16 + 8) == INVALID  # misaligned
    assert call(eps=-1.0) == INVALID
    assert call(eps=float("nan")) == INVALID
    assert call(Bn=0) == INVALID


def test_layer_noalloc_rejects_bad_arguments_and_large_shapes():
    # every case fails validation or the scratch-size check, both before any HIP call
    P, W = pred(F=1024), ffn(F=1024)
    call = lambda P=P, W=W, x=None, Bn=1, idx=None, y=None: lib.psffn_layer_noalloc(
        B(P), B(W), fake() if x is None else x, Bn, 0.0, fake() if idx is None else idx, fake(), None,
        fake() if y is None else y, 0, None)
    assert lib.psffn_layer_noalloc(None, B(W), fake(), 1, 0.0, fake(), fake(), None, fake(), 0, None) == INVALID
    assert call(P=pred(F=2048)) == INVALID  # P and W describe different layers
    assert call(P=pred(F=1024, dt=ps.PSFFN_F32)) == UNSUPPORTED  # fp32 predictor with fp16 weights
    assert call(Bn=0) == INVALID
    assert call(Bn=ps.MAX_BATCH + 1) == INVALID
    assert call(x=A16 + 4) == INVALID
    assert call(idx=A16 + 2) == INVALID
    # a layer whose workspace exceeds the static scratch (PSFFN_NOALLOC_SCRATCH_BYTES = 64 MiB)
    big_p = pred(d=12288, F=49152, r=1536)
    big_w = ffn(d=12288, F=49152, dt=ps.PSFFN_I4G128)
    assert lib.psffn_workspace_bytes(B(big_p), B(big_w), 32) > (64 << 20)
    assert call(P=big_p, W=big_w, Bn=32) == WORKSPACE
