"""Seeded synthetic inputs for the routed MoE FFN layer.

This module only draws and stores inputs; it holds none of the layer's
arithmetic (no routing, no expert evaluation, no combine).  Both the GPU
path (through the tests and the bench) and the CPU oracle receive the
same tensors from here.

Distributions (the shapes come from the pages' statement of the layer:
D = 4096, E = 512 experts of I = 1024, top-10, one shared expert; the
512-request decode batch and the 8K prefill chunk are the pages' serving
shapes):

* hidden states x ~ N(0, 1);
* router W_r [E][D], W_gate / W_up [E][I][D] with std 1/sqrt(D);
  W_down [E][D][I] with std 1/sqrt(I); the shared expert likewise;
* bf16 workloads round the float32 draws to bf16 (torch's cast, round to
  nearest even); the fp32 workload keeps the float32 draws;
* fp8 weights: per output channel c, the draw z is mapped to E4M3 codes
  as cast(z * 448 / amax_c) (torch's cast, after a clamp to +-448) with
  an fp32 scale amax_c / 448 * std, so code * scale ~ N(0, std^2);
* skewed routing: a per-expert additive logit bias
  b_e = -alpha * s * ln(r_e) with r a seeded random ranking 1..E of the
  experts (a Zipf(s) popularity), plus b_e = -inf for the n_empty lowest
  ranked experts, which therefore receive no token;
* given routing (one device's expert-parallel share): per token, k
  distinct experts drawn uniformly without replacement and weights drawn
  as normalised exponentials sorted in descending order, stored as the
  packed [T][2][k] int32 blob (ids, fp32 weight bits).

Small workloads are drawn on the host with NumPy (PCG64 keyed by
(seed, tensor id, expert id)), so the CPU-only tests see exactly the same
values everywhere.  Full-size workloads (12.9 GB of bf16 weights) are
drawn on the GPU with torch's Philox generator keyed the same way; the
oracle reads back from the device only the experts it needs.
"""

from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Optional

import numpy as np

try:
    import torch
except ImportError:  # pragma: no cover - torch is part of the image
    torch = None


# ---------------------------------------------------------------------------
# Workloads
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    D: int
    E: int
    top_k: int
    I: int
    I_shared: int          # 0: no shared expert
    act: str               # "f32" | "bf16"
    w: str                 # "f32" | "bf16" | "e4m3"
    out: str               # "f32" | "bf16"
    expert_begin: int = 0
    n_local: Optional[int] = None
    skew_alpha: Optional[float] = None   # Zipf bias strength (None: no bias)
    skew_s: float = 1.1
    skew_empty: int = 0
    routing_given: bool = False          # routing arrives as a packed blob
    renormalize: bool = True

    @property
    def local(self) -> int:
        return self.E if self.n_local is None else self.n_local

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    # Tiny fp32 layer: correctness at launch-latency scale.
    "tiny_fp32": Workload("tiny_fp32", T=64, D=256, E=16, top_k=2, I=128, I_shared=128,
                          act="f32", w="f32", out="f32"),
    # 512 concurrent requests, one token each: weight streaming.
    "decode_bf16": Workload("decode_bf16", T=512, D=4096, E=512, top_k=10, I=1024, I_shared=1024,
                            act="bf16", w="bf16", out="bf16"),
    # An 8K-token prefill chunk of the same layer.
    "prefill_bf16": Workload("prefill_bf16", T=8192, D=4096, E=512, top_k=10, I=1024, I_shared=1024,
                             act="bf16", w="bf16", out="bf16"),
    # The prefill chunk with Zipf-skewed expert popularity and 32 never-chosen experts.
    "skew_prefill_bf16": Workload("skew_prefill_bf16", T=8192, D=4096, E=512, top_k=10, I=1024,
                                  I_shared=1024, act="bf16", w="bf16", out="bf16",
                                  skew_alpha=0.36, skew_s=1.1, skew_empty=32),
    # One device's expert-parallel share: 8 x 1024 gathered tokens, local experts 0..63, e4m3 weights.
    "ep_share_fp8": Workload("ep_share_fp8", T=8192, D=4096, E=512, top_k=10, I=1024, I_shared=0,
                             act="bf16", w="e4m3", out="bf16", expert_begin=0, n_local=64,
                             routing_given=True),
    # A 32K-token prefill chunk (~640 rows per expert): large enough for the grouped GEMMs
    # to be MFMA-bound rather than weight-stream bound; a supplementary probe.
    "prefill32k_bf16": Workload("prefill32k_bf16", T=32768, D=4096, E=512, top_k=10, I=1024, I_shared=1024,
                                act="bf16", w="bf16", out="bf16"),
    # The decode batch with the routed experts stored as e4m3 codes + per-channel fp32 scales
    # (about one byte per parameter); router and shared expert stay bf16.
    "decode_fp8": Workload("decode_fp8", T=512, D=4096, E=512, top_k=10, I=1024, I_shared=1024,
                           act="bf16", w="e4m3", out="bf16"),
}


# ---------------------------------------------------------------------------
# Seeding
# ---------------------------------------------------------------------------

_TID = {"x": 1, "w_router": 2, "w_gate": 3, "w_up": 4, "w_down": 5,
        "ws_gate": 6, "ws_up": 7, "ws_down": 8, "bias_rank": 9, "routing": 10}


def _key(seed: int, tensor: str, sub: int = 0) -> np.random.SeedSequence:
    return np.random.SeedSequence([seed, _TID[tensor], sub])


def _torch_seed(seed: int, tensor: str, sub: int = 0) -> int:
    return int(_key(seed, tensor, sub).generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))


_TORCH_DT = {}
if torch is not None:
    _TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "e4m3": torch.float8_e4m3fn}


# ---------------------------------------------------------------------------
# Drawing
# ---------------------------------------------------------------------------

def _normal_host(seed, tensor, sub, shape, std):
    rng = np.random.Generator(np.random.PCG64(_key(seed, tensor, sub)))
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def _normal_dev(seed, tensor, sub, shape, std, device):
    g = torch.Generator(device=device)
    g.manual_seed(_torch_seed(seed, tensor, sub))
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std


def _store(z: "torch.Tensor", dt: str) -> "torch.Tensor":
    """float32 draws -> storage dtype (f32 kept, bf16 by torch's RNE cast)."""
    return z if dt == "f32" else z.to(_TORCH_DT[dt])


def _fp8_channels(z: "torch.Tensor"):
    """float32 draws [out, in] (already scaled by the weight std) -> (E4M3 codes [out, in], fp32 scale
    per output channel [out]), so that codes * scale ~ z: each channel's largest magnitude maps to 448."""
    amax = z.abs().amax(dim=1, keepdim=True).clamp_min(1e-30)
    codes = (z * (448.0 / amax)).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    scale = (amax[:, 0] / 448.0).to(torch.float32)
    return codes, scale


def zipf_bias(E: int, alpha: float, s: float, n_empty: int, seed: int) -> np.ndarray:
    """Per-expert fp32 logit bias: -alpha * s * ln(rank), and -inf for the n_empty lowest ranks."""
    rng = np.random.Generator(np.random.PCG64(_key(seed, "bias_rank")))
    rank = rng.permutation(E) + 1                      # expert e has popularity rank rank[e]
    b = (-alpha * s * np.log(rank.astype(np.float64))).astype(np.float32)
    if n_empty:
        b[rank > E - n_empty] = -np.inf
    return b


def given_routing(T: int, E: int, k: int, seed: int) -> np.ndarray:
    """Packed [T][2][k] blob: k distinct uniform experts per token, weights sorted descending, sum ~ 1."""
    rng = np.random.Generator(np.random.PCG64(_key(seed, "routing")))
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    w = rng.standard_exponential((T, k))
    w = -np.sort(-(w / w.sum(axis=1, keepdims=True)), axis=1)
    w32 = np.ascontiguousarray(w.astype(np.float32))
    return np.stack([ids, w32.view(np.int32)], axis=1)


@dataclass
class LayerInputs:
    """The layer's tensors in their storage dtypes (torch, on one device)."""
    wl: Workload
    x: "torch.Tensor"                      # [T, D] act dtype
    w_router: Optional["torch.Tensor"]     # [E, D] act dtype (None when routing is given)
    w_gate: "torch.Tensor"                 # [n_local, I, D]
    w_up: "torch.Tensor"                   # [n_local, I, D]
    w_down: "torch.Tensor"                 # [n_local, D, I]
    s_gate: Optional["torch.Tensor"] = None    # [n_local, I] fp32 (e4m3 only)
    s_up: Optional["torch.Tensor"] = None      # [n_local, I]
    s_down: Optional["torch.Tensor"] = None    # [n_local, D]
    ws_gate: Optional["torch.Tensor"] = None   # [I_s, D] shared expert
    ws_up: Optional["torch.Tensor"] = None
    ws_down: Optional["torch.Tensor"] = None   # [D, I_s]
    bias: Optional["torch.Tensor"] = None      # [E] fp32
    packed: Optional["torch.Tensor"] = None    # [T, 2, k] int32

    def to(self, device) -> "LayerInputs":
        kw = {f.name: getattr(self, f.name) for f in dataclasses.fields(self)}
        for k_, v in kw.items():
            if torch is not None and isinstance(v, torch.Tensor):
                kw[k_] = v.to(device)
        return LayerInputs(**kw)


def make_inputs(wl: Workload, seed: int = 0, device: str = "cpu") -> LayerInputs:
    """Draw every input of workload ``wl``.

    device "cpu": NumPy draws (bit-identical on any machine), returned as
    CPU tensors.  Any other device: torch Philox draws made on that
    device (used for the full-size workloads).
    """
    T, D, E, I, Is, nl = wl.T, wl.D, wl.E, wl.I, wl.I_shared, wl.local
    on_host = str(device) == "cpu"

    def normal(tensor, sub, shape, std):
        if on_host:
            return torch.from_numpy(_normal_host(seed, tensor, sub, shape, std))
        return _normal_dev(seed, tensor, sub, shape, std, device)

    x = _store(normal("x", 0, (T, D), 1.0), wl.act)
    w_router = None if wl.routing_given else _store(normal("w_router", 0, (E, D), D ** -0.5), wl.act)

    def expert_stack(tensor, shape, std):
        if wl.w == "e4m3":
            codes, scales = [], []
            for e in range(nl):
                c, s = _fp8_channels(normal(tensor, wl.expert_begin + e, shape, std))
                codes.append(c)
                scales.append(s)
            return torch.stack(codes), torch.stack(scales)
        out = torch.empty((nl,) + shape, dtype=_TORCH_DT[wl.w], device=device)
        for e in range(nl):
            out[e] = _store(normal(tensor, wl.expert_begin + e, shape, std), wl.w)
        return out, None

    w_gate, s_gate = expert_stack("w_gate", (I, D), D ** -0.5)
    w_up, s_up = expert_stack("w_up", (I, D), D ** -0.5)
    w_down, s_down = expert_stack("w_down", (D, I), I ** -0.5)

    ws_gate = ws_up = ws_down = None
    if Is:
        sdt = wl.act if wl.w == "e4m3" else wl.w
        ws_gate = _store(normal("ws_gate", 0, (Is, D), D ** -0.5), sdt)
        ws_up = _store(normal("ws_up", 0, (Is, D), D ** -0.5), sdt)
        ws_down = _store(normal("ws_down", 0, (D, Is), Is ** -0.5), sdt)

    bias = None
    if wl.skew_alpha is not None:
        bias = torch.from_numpy(zipf_bias(E, wl.skew_alpha, wl.skew_s, wl.skew_empty, seed + 1)).to(device)
    packed = None
    if wl.routing_given:
        packed = torch.from_numpy(given_routing(T, E, wl.top_k, seed)).to(device)

    return LayerInputs(wl, x, w_router, w_gate, w_up, w_down, s_gate, s_up, s_down,
                       ws_gate, ws_up, ws_down, bias, packed)


# ---------------------------------------------------------------------------
# Views for the oracle (storage dtype -> exact float64 images)
# ---------------------------------------------------------------------------

def f64(t) -> np.ndarray:
    """Exact float64 image of a stored tensor (any device)."""
    if t is None:
        return None
    return t.detach().to("cpu").to(torch.float64).numpy()


class ExpertView:
    """experts[e] -> (w_gate, w_up, w_down) as float64 for local expert e, fetched on demand."""

    def __init__(self, inp: LayerInputs):
        self.inp = inp

    def __len__(self):
        return self.inp.w_gate.shape[0]

    def __getitem__(self, e):
        i = self.inp
        return f64(i.w_gate[e]), f64(i.w_up[e]), f64(i.w_down[e])


class ExpertViewFP8:
    """experts[e] -> ((g codes, g scale), (u codes, u scale), (d codes, d scale)) in float64."""

    def __init__(self, inp: LayerInputs):
        self.inp = inp

    def __len__(self):
        return self.inp.w_gate.shape[0]

    def __getitem__(self, e):
        i = self.inp
        return ((f64(i.w_gate[e]), f64(i.s_gate[e])),
                (f64(i.w_up[e]), f64(i.s_up[e])),
                (f64(i.w_down[e]), f64(i.s_down[e])))


def shared_f64(inp: LayerInputs):
    if inp.ws_gate is None:
        return None
    return f64(inp.ws_gate), f64(inp.ws_up), f64(inp.ws_down)
