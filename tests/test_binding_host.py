"""Argument checks of the Python binding (no GPU, no library call is reached): the C ABI sees only
raw pointers, so the binding rejects tensors whose dtype, shape, contiguity or device would make a
kernel read or write outside a buffer, with ValueError, before calling into the library."""
import pytest
import torch

ps = pytest.importorskip("activation_sparse_ffn_psffn_amd")

d, F, r = 64, 96, 16


def f16(*s):
    return torch.zeros(*s, dtype=torch.float16)


def f32(*s):
    return torch.zeros(*s, dtype=torch.float32)


def i32(*s):
    return torch.zeros(*s, dtype=torch.int32)


def layer_parts(w=torch.float16):
    P = ps.Predictor(torch.zeros(r, d, dtype=w), torch.zeros(F, r, dtype=w), f32(F))
    W = ps.FFN("relu", torch.zeros(F, d, dtype=w), torch.zeros(F, d, dtype=w), b_up=f32(F))
    return P, W


def raises(fn, match):
    with pytest.raises(ValueError, match=match):
        fn()


def test_descriptor_checks():
    P, W = layer_parts()
    raises(lambda: ps.Predictor(f16(r, d), f16(F, r + 8), f32(F)).struct(), "Predictor.Q")
    raises(lambda: ps.Predictor(f16(r, d), torch.zeros(F, r), f32(F)).struct(), "Predictor.Q")  # dtype differs
    raises(lambda: ps.Predictor(f16(r, d), f16(F, r), f16(F)).struct(), "Predictor.c")
    raises(lambda: ps.Predictor(f16(d, r).t(), f16(F, r), f32(F)).struct(), "contiguous")
    raises(lambda: ps.FFN("relu", f16(F, d), f16(F, d + 8)).struct(), "w_dT")
    raises(lambda: ps.FFN("relu", f16(F, d), torch.zeros(F, d)).struct(), "w_dT")
    raises(lambda: ps.FFN("swiglu", f16(F, d), f16(F, d)).struct(), "w_gate")
    raises(lambda: ps.FFN("gelu", f16(F, d), f16(F, d)).struct(), "act")
    raises(lambda: ps.FFN("relu", f16(F, d), f16(F, d), b_up=f32(F + 1)).struct(), "b_up")
    raises(lambda: ps.FFN("relu", f16(F, d), f16(F, d), b_down=f32(F)).struct(), "b_down")
    raises(lambda: ps.FFN("relu", torch.zeros(F, d, dtype=torch.int8), f16(F, d)).struct(), "uint8")
    # 4-bit: packed rows [F][d/2] with fp16 scales [F][d/128]
    q = torch.zeros(F, 128, dtype=torch.uint8)
    raises(lambda: ps.FFN("relu", q, q).struct(), "s_up")
    raises(lambda: ps.FFN("relu", q, q, s_up=f16(F, 2), s_dT=f16(F, 1)).struct(), "s_dT")
    # a CPU tensor of the right type and shape is still refused: the library takes device pointers
    raises(lambda: P.struct(), "GPU tensor")
    raises(lambda: W.struct(), "GPU tensor")


def test_call_argument_checks():
    P, W = layer_parts()
    ws = torch.zeros(1 << 16, dtype=torch.uint8)
    x = f16(1, d)
    # activation dtype follows the weights (fp16 here), shapes follow the layer
    raises(lambda: ps._batch(torch.zeros(1, d), d, W.act_dtype), "dtype")
    raises(lambda: ps._batch(f16(1, d + 8), d, W.act_dtype), "shape")
    raises(lambda: ps._batch(f16(ps.MAX_BATCH + 1, d), d, W.act_dtype), "batch")
    raises(lambda: ps._batch(f16(0, d), d, W.act_dtype), "batch")
    raises(lambda: ps._batch(f16(d, 2).t(), d, W.act_dtype), "contiguous")
    raises(lambda: ps._batch(f16(d), d, W.act_dtype), r"\[B\]\[d\]")
    # outputs: int32 list with room for F entries, fp32 y [B][d], fp32 logits [B][F], uint8 workspace
    raises(lambda: ps._outs(x.device, F, torch.zeros(F, dtype=torch.int64), None), "idx")
    raises(lambda: ps._outs(x.device, F, i32(F - 1), None), "idx")
    raises(lambda: ps._outs(x.device, F, None, torch.zeros(1, dtype=torch.int64)), "count")
    raises(lambda: ps._outs(x.device, F, None, None, f32(1, F + 1), 1), "logits")
    raises(lambda: ps._outs(x.device, F, None, None, B=1, y=f16(1, d), d=d), "y")
    raises(lambda: ps._outs(x.device, F, None, None, B=1, y=f32(2, d), d=d), "y")
    raises(lambda: ps._outs(x.device, F, None, None, ws=torch.zeros(64, dtype=torch.float32)), "ws")
    # whole calls stop in the binding (CPU tensors, or wrong types) before the library is reached
    raises(lambda: ps.predict(P, x, ws), "GPU tensor")
    raises(lambda: ps.layer(P, W, x, ws), "GPU tensor")
    raises(lambda: ps.sparse_ffn(W, x, i32(F), i32(1), ws), "GPU tensor")
    raises(lambda: ps.layer_ln(P, W, f16(1, d), ws), "GPU tensor")
    raises(lambda: ps.layernorm_f16(f16(1, d)), "dtype")
    raises(lambda: ps.compact(f32(F), ws), r"\[B\]\[F\]")
    raises(lambda: ps.permute_hot_first(torch.zeros(F, dtype=torch.int64)), "counts")
    raises(lambda: ps.workspace_init(torch.zeros(64)), "ws")


def test_layer_pair_checks():
    P, _ = layer_parts()
    W2 = ps.FFN("relu", f16(F + 8, d), f16(F + 8, d))
    raises(lambda: ps._pair(P, W2), "different layers")
