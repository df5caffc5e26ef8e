"""Seeded synthetic inputs for the predictor-gated sparse FFN.

This module only BUILDS inputs: weight matrices, biases, predictor weights, decode tokens and
profiling tokens.  It holds none of the method's arithmetic (no prediction, no thresholding,
no compaction, no FFN, no dequantisation on the compute side) and is shared by the CPU oracle
tests and the HIP tests / benchmark, which then both read the same bytes.

Workloads (power-law neuron firing, "PowerInfer: Fast Large Language Model Serving with a
Consumer-grade GPU", Elamur Research summary, Summary, 1st paragraph: a few hot neurons fire
for most inputs, a long tail of cold ones only for some; Key points: OPT-30B's ReLU MLP is
97% sparse, LLaMA2-13B's SwiGLU MLP 43%).  The pages print no weights, so the layers are
random with the model shapes and those sparsities:

* weights W ~ N(0, 1/d), rounded to the storage type (fp32, fp16, or 4-bit groups);
* neuron firing probabilities p follow a Zipf law in a random rank order, scaled to the
  layer's mean density and clipped at 0.999;
* the bias of neuron i is b_i = ||w_i|| * Phi^-1(p_i) with ||w_i|| the norm of the STORED row,
  so that for x ~ N(0, I) the pre-activation w_i.x + b_i is > 0 with probability exactly p_i;
* the predictor is low rank, l = Q (A x) + c with A [r][d], Q [F][r] ~ N(0, 1/d) and
  c_i = ||A^T q_i|| * Phi^-1(p_i), the same construction, so P(l_i > 0) = p_i as well.

Random numbers come from torch generators seeded per (seed, layer, tensor): a tensor does not
depend on the order in which tensors are drawn.  The CPU and GPU generators produce different
streams; every test draws its inputs once and hands the same bytes to both sides.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np
import torch

P_MAX = 0.999  # clip of the Zipf firing probabilities (an unclipped Zipf law exceeds 1)


@dataclass(frozen=True)
class LayerSpec:
    name: str
    d: int
    F: int
    r: int
    storage: str  # "f32" | "f16" | "i4"  (4-bit weights, fp16 predictor and activations)
    act: str  # "relu" | "swiglu"
    density: float
    zipf: float
    tokens: int
    batches: tuple = (1,)
    hot_first: bool = False
    profile_tokens: int = 0
    layers: int = 1
    density_range: Optional[tuple] = None  # per-layer density drawn uniformly from this range
    group: int = 128


CONFIGS = {
    "tiny_relu_f32": LayerSpec("tiny_relu_f32", d=256, F=1024, r=32, storage="f32", act="relu", density=0.10,
                               zipf=1.1, tokens=64),
    "opt30b_relu_f16": LayerSpec("opt30b_relu_f16", d=7168, F=28672, r=1024, storage="f16", act="relu",
                                 density=0.03, zipf=1.1, tokens=1024, hot_first=True, profile_tokens=512),
    "llama2_13b_swiglu_f16": LayerSpec("llama2_13b_swiglu_f16", d=5120, F=13824, r=1024, storage="f16",
                                       act="swiglu", density=0.57, zipf=0.8, tokens=1024),
    "opt175b_relu_i4": LayerSpec("opt175b_relu_i4", d=12288, F=49152, r=1536, storage="i4", act="relu",
                                 density=0.03, zipf=1.1, tokens=1024, batches=(1, 8)),
    "falcon40b_stack_f16": LayerSpec("falcon40b_stack_f16", d=8192, F=32768, r=1024, storage="f16", act="relu",
                                     density=0.06, zipf=1.0, tokens=256, batches=(1, 4, 32), layers=48,
                                     density_range=(0.02, 0.10)),
}

_TAGS = {"w_up": 1, "w_gate": 2, "w_dT": 3, "A": 4, "Q": 5, "rank": 6, "tokens": 7, "profile": 8, "density": 9,
         "x0": 10, "aligned": 11}


def _gen(seed: int, layer: int, tag: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    key = (int(seed) * 1_000_003 + int(layer) * 10_007 + _TAGS[tag] * 101 + 17) % (2 ** 62)
    g.manual_seed(key)
    return g


def zipf_firing_probs(F: int, s: float, density: float, p_max: float = P_MAX) -> np.ndarray:
    """Firing probability of the neuron of Zipf rank k = 1..F: p_k = min(p_max, kappa k^-s),
    with kappa found by fp64 bisection so that the mean of p is `density`."""
    q = np.arange(1, F + 1, dtype=np.float64) ** (-float(s))
    if not (0.0 < density < p_max):
        raise ValueError("density must lie in (0, p_max)")
    lo, hi = 0.0, p_max / q[-1]  # at hi every p is clipped -> mean p_max > density
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if np.minimum(p_max, mid * q).mean() < density:
            lo = mid
        else:
            hi = mid
    return np.minimum(p_max, 0.5 * (lo + hi) * q)


def layer_density(spec: LayerSpec, seed: int, layer: int) -> float:
    if spec.density_range is None:
        return spec.density
    g = _gen(seed, layer, "density", "cpu")
    u = torch.rand(1, generator=g, dtype=torch.float64).item()
    lo, hi = spec.density_range
    return lo + (hi - lo) * u


def neuron_probs(spec: LayerSpec, seed: int, layer: int = 0) -> np.ndarray:
    """p[i] for neuron i: Zipf ranks assigned to neurons by a seeded random permutation."""
    pz = zipf_firing_probs(spec.F, spec.zipf, layer_density(spec, seed, layer))
    rank_of = torch.randperm(spec.F, generator=_gen(seed, layer, "rank", "cpu")).numpy()
    return pz[rank_of]


def _normal(shape, scale, g, device):
    return torch.randn(*shape, generator=g, device=device, dtype=torch.float32) * scale


def _store(w32: torch.Tensor, storage: str) -> torch.Tensor:
    return w32 if storage == "f32" else w32.to(torch.float16)


def quantize_i4_g128(w32: torch.Tensor, group: int = 128):
    """Encode a float matrix [F][d] as 4-bit groups: per `group` consecutive elements of a row,
    scale s = fp16(max|w| / 7) and q = clamp(round-half-even(w / s), -8, 7) in two's complement;
    element 2j in the low nibble of byte j, element 2j+1 in the high nibble.
    Returns (packed uint8 [F][d/2], scales float16 [F][d/group], the exact values q*s as fp64)."""
    F, d = w32.shape
    assert d % group == 0 and d % 2 == 0
    wg = w32.reshape(F, d // group, group)
    s16 = (wg.abs().amax(-1) / 7.0).to(torch.float16)
    s32 = s16.to(torch.float32)
    safe = torch.where(s32 > 0, s32, torch.ones_like(s32))
    q = torch.round(wg / safe[..., None]).clamp_(-8, 7)
    q = torch.where(s32[..., None] > 0, q, torch.zeros_like(q)).to(torch.int16).reshape(F, d)
    nib = (q & 15).to(torch.uint8)
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).contiguous()
    exact = q.to(torch.float64).reshape(F, d // group, group) * s16.to(torch.float64)[..., None]
    return packed, s16.contiguous(), exact.reshape(F, d)


def _row_norm64(w: torch.Tensor) -> torch.Tensor:
    out = torch.empty(w.shape[0], dtype=torch.float64, device=w.device)
    step = max(1, (1 << 26) // max(1, w.shape[1]))
    for i in range(0, w.shape[0], step):
        out[i:i + step] = w[i:i + step].to(torch.float64).norm(dim=1)
    return out


def _bias(norms64: torch.Tensor, p: np.ndarray) -> torch.Tensor:
    z = torch.special.ndtri(torch.from_numpy(p).to(norms64.device))
    return (norms64 * z).to(torch.float32).contiguous()


@dataclass
class Layer:
    """One layer's tensors, all on `device`, neuron-major (row i of every [F][.] tensor is neuron i)."""
    spec: LayerSpec
    w_up: torch.Tensor
    w_dT: torch.Tensor
    A: torch.Tensor
    Q: torch.Tensor
    c: torch.Tensor
    p: np.ndarray
    w_gate: Optional[torch.Tensor] = None
    s_up: Optional[torch.Tensor] = None
    s_gate: Optional[torch.Tensor] = None
    s_dT: Optional[torch.Tensor] = None
    b_up: Optional[torch.Tensor] = None
    b_gate: Optional[torch.Tensor] = None
    b_down: Optional[torch.Tensor] = None
    extra: dict = field(default_factory=dict)

    def numpy(self) -> dict:
        """Host copies of every tensor (the same bytes), keyed by name."""
        out = {}
        for k in ("w_up", "w_gate", "w_dT", "s_up", "s_gate", "s_dT", "b_up", "b_gate", "b_down", "A", "Q", "c"):
            t = getattr(self, k)
            out[k] = None if t is None else t.detach().cpu().contiguous().numpy()
        return out

    def permuted(self, perm: torch.Tensor) -> "Layer":
        """Host-side reference reordering (new neuron k = old neuron perm[k]) -- input plumbing
        for tests that need a permuted layer without going through the library."""
        pm = perm.to(self.w_up.device).long()
        g = lambda t: None if t is None else t[pm].contiguous()
        return replace(self, w_up=g(self.w_up), w_dT=g(self.w_dT), w_gate=g(self.w_gate), s_up=g(self.s_up),
                       s_gate=g(self.s_gate), s_dT=g(self.s_dT), b_up=g(self.b_up), b_gate=g(self.b_gate),
                       Q=g(self.Q), c=g(self.c), p=self.p[perm.cpu().numpy()])


def make_layer(spec: LayerSpec, seed: int = 0, layer: int = 0, device="cpu", d: int = None, F: int = None,
               r: int = None) -> Layer:
    """Build one layer of `spec` (optionally with overridden sizes for small test shapes)."""
    d = d or spec.d
    F = F or spec.F
    r = r or spec.r
    if (d, F, r) != (spec.d, spec.F, spec.r):
        spec = replace(spec, d=d, F=F, r=r)
    p = neuron_probs(spec, seed, layer)
    scale = 1.0 / math.sqrt(d)
    pstore = "f32" if spec.storage == "f32" else "f16"
    L = {}
    gates = ("w_up", "w_gate") if spec.act == "swiglu" else ("w_up",)
    biased = "w_gate" if spec.act == "swiglu" else "w_up"  # the branch that decides firing
    for name in gates + ("w_dT",):
        w32 = _normal((F, d), scale, _gen(seed, layer, name, device), device)
        if spec.storage == "i4":
            packed, s16, exact = quantize_i4_g128(w32, spec.group)
            L[name] = packed
            L["s" + name[1:]] = s16
            norms = exact.norm(dim=1) if name == biased else None
        else:
            L[name] = _store(w32, spec.storage).contiguous()
            norms = _row_norm64(L[name]) if name == biased else None
        if norms is not None:
            L["b" + name[1:]] = _bias(norms, p)
        del w32
    A = _store(_normal((r, d), scale, _gen(seed, layer, "A", device), device), pstore).contiguous()
    Q = _store(_normal((F, r), scale, _gen(seed, layer, "Q", device), device), pstore).contiguous()
    A64 = A.to(torch.float64)
    G = A64 @ A64.T  # r x r
    Q64 = Q.to(torch.float64)
    var = ((Q64 @ G) * Q64).sum(dim=1).clamp_min(0.0)
    c = _bias(var.sqrt(), p)
    del A64, G, Q64
    return Layer(spec=spec, w_up=L["w_up"], w_dT=L["w_dT"], w_gate=L.get("w_gate"), s_up=L.get("s_up"),
                 s_gate=L.get("s_gate"), s_dT=L.get("s_dT"), b_up=L.get("b_up"), b_gate=L.get("b_gate"), A=A, Q=Q,
                 c=c, p=p)


def make_aligned_predictor(L: Layer, r: int, seed: int = 0):
    """A predictor ALIGNED with the layer (input construction for the predictor-accuracy study).

    The layer's deciding branch W (W_up for ReLU, W_gate for SwiGLU; dense storage only) is
    approximated at rank r, W ~= U_r S_r V_r^T, by a seeded randomized range finder with two power
    iterations; the predictor is A = V_r^T [r][d], Q = U_r S_r [F][r] and c = the branch's bias,
    stored in the predictor's type, so l = Q (A x) + c approximates the true pre-activation.  The
    generated predictor of make_layer is instead independent of W (equal firing rates only).
    Returns (A, Q, c) on the layer's device."""
    if L.spec.storage == "i4":
        raise ValueError("make_aligned_predictor: dense layers only")
    W = (L.w_gate if L.spec.act == "swiglu" else L.w_up).to(torch.float32)
    bias = L.b_gate if L.spec.act == "swiglu" else L.b_up
    F, d = W.shape
    q = min(r + 16, d, F)
    g = _gen(seed, r, "aligned", W.device)
    Y = W @ torch.randn(d, q, generator=g, device=W.device, dtype=torch.float32)
    for _ in range(2):
        Y, _ = torch.linalg.qr(Y)
        Y = W @ (W.T @ Y)
    Qb, _ = torch.linalg.qr(Y)  # F x q orthonormal basis of W's dominant range
    U_s, S, Vh = torch.linalg.svd(Qb.T @ W, full_matrices=False)  # (q x d) = U_s S Vh
    U = Qb @ U_s[:, :r]
    pstore = "f32" if L.spec.storage == "f32" else "f16"
    A = _store(Vh[:r].contiguous(), pstore).contiguous()
    Qm = _store((U * S[:r]).contiguous(), pstore).contiguous()
    c = (bias if bias is not None else torch.zeros(F, device=W.device)).to(torch.float32).contiguous()
    return A, Qm, c


def make_tokens(spec: LayerSpec, n: int, seed: int = 0, stream: str = "tokens", device="cpu", d: int = None):
    """n decode tokens x ~ N(0, I) in the activation storage type (fp32 for fp32 layers, else fp16).
    stream="profile" gives the independent profiling tokens."""
    d = d or spec.d
    x = torch.randn(n, d, generator=_gen(seed, 0, stream, device), device=device, dtype=torch.float32)
    return x if spec.storage == "f32" else x.to(torch.float16)


def make_residual(spec: LayerSpec, n: int, seed: int = 0, device="cpu", d: int = None):
    """Initial fp32 residual stream of the decode stack, x0 ~ N(0, I)."""
    d = d or spec.d
    return torch.randn(n, d, generator=_gen(seed, 0, "x0", device), device=device, dtype=torch.float32)


def profile_like_counts(p: np.ndarray, T: int, seed: int = 0) -> np.ndarray:
    """Synthetic fire counts with the statistics of a T-token profile: counts_i ~ Binomial(T, p_i),
    int32.  An input for the hot-first order that does not depend on any implementation."""
    g = torch.Generator().manual_seed(int(seed) * 7919 + 3)
    pt = torch.from_numpy(np.asarray(p, dtype=np.float64)).to(torch.float32)
    c = torch.binomial(torch.full_like(pt, float(T)), pt, generator=g)
    return c.to(torch.int32).numpy()
