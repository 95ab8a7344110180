"""Run the GPU library and the CPU oracle on the same seeded inputs.

Test infrastructure: imports both the binding and the oracle (the two never
import each other).
"""

from __future__ import annotations

import numpy as np
import torch

import oracle
import sparse_moe_ffn_route_amd as moe
import synth

_OUT_TORCH = {"f32": torch.float32, "bf16": torch.bfloat16}


def dims_of(wl: synth.Workload, shared: bool = True, packed: bool = False) -> moe.moe_dims:
    return moe.make_dims(wl.T, wl.D, wl.E, wl.top_k, wl.I, wl.I_shared if shared else 0, wl.expert_begin,
                         wl.local, wl.renormalize, wl.act, wl.w, wl.out, "packed" if packed else "rows")


def packed_weights(dev: synth.LayerInputs) -> dict:
    """Expert and shared weights repacked on the GPU by moe_pack_weights."""
    out = {}
    for name in ("w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down"):
        t = getattr(dev, name)
        out[name] = None if t is None else moe.moe_pack_weights(t)
    return out


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def gpu_layer(inp: synth.LayerInputs, shared: bool = True, ws: torch.Tensor = None, packed: bool = False) -> dict:
    """moe_layer_forward on the inputs (moved to the GPU); returns host copies."""
    wl = inp.wl
    dev = inp if inp.x.is_cuda else inp.to("cuda")
    d = dims_of(wl, shared, packed)
    y = torch.empty(wl.T, wl.D, dtype=_OUT_TORCH[wl.out], device="cuda")
    logits = None if wl.routing_given else torch.empty(wl.T, wl.E, dtype=torch.float32, device="cuda")
    blob = torch.empty(wl.T, 2, wl.top_k, dtype=torch.int32, device="cuda")
    if ws is None:
        ws = moe.workspace(d)
    use_shared = shared and wl.I_shared > 0
    pw = packed_weights(dev) if packed else {n: getattr(dev, n) for n in
                                             ("w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down")}
    w = moe.make_weights(dev.w_router, pw["w_gate"], pw["w_up"], pw["w_down"], dev.s_gate, dev.s_up, dev.s_down,
                         pw["ws_gate"] if use_shared else None, pw["ws_up"] if use_shared else None,
                         pw["ws_down"] if use_shared else None)
    moe.moe_layer_forward(d, w, dev.x, dev.packed, dev.bias, y, logits, blob, ws)
    torch.cuda.synchronize()
    return dict(y=to_np(y), logits=None if logits is None else logits.cpu().numpy(),
                packed=blob.cpu().numpy(), dev=dev)


def oracle_routing(inp: synth.LayerInputs, logits=None):
    """(ids, weights) the oracle derives: from the given blob, or from these fp32 logits."""
    wl = inp.wl
    if wl.routing_given:
        ids, w32 = oracle.unpack_routing(inp.packed.cpu().numpy())
        return ids, w32.astype(np.float64)
    bias = None if inp.bias is None else inp.bias.cpu().numpy()
    return oracle.route(logits, wl.top_k, bias=bias, renormalize=wl.renormalize)


def oracle_layer(inp: synth.LayerInputs, logits=None, shared: bool = True) -> dict:
    wl = inp.wl
    ids, w = oracle_routing(inp, logits)
    x = synth.f64(inp.x)
    if wl.w == "e4m3":
        sh = synth.shared_f64(inp) if shared else None
        res = oracle.layer_from_routing_fp8(x, ids, w, synth.ExpertViewFP8(inp), shared=sh,
                                            expert_begin=wl.expert_begin, n_local=wl.local)
    else:
        sh = synth.shared_f64(inp) if shared else None
        res = oracle.layer_from_routing(x, ids, w, synth.ExpertView(inp), shared=sh,
                                        expert_begin=wl.expert_begin, n_local=wl.local)
    res.update(ids=ids, weights=w)
    return res


def logit_bound(x: np.ndarray, w_router: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Worst-case fp32 accumulation error of a D-term dot product of exact products, plus the final rounding."""
    D = x.shape[1]
    mag = np.abs(x) @ np.abs(w_router).T
    return D * 2.0 ** -24 * mag + 2.0 ** -24 * np.abs(ref)


def rel_err(y: np.ndarray, y_ref: np.ndarray) -> float:
    scale = np.abs(y_ref).max()
    return float(np.abs(y - y_ref).max() / (scale if scale > 0 else 1.0))


TOL = {"f32": 1e-4, "bf16": 1e-2, "e4m3": 3e-2}


def tolerance(wl: synth.Workload) -> float:
    return TOL["e4m3"] if wl.w == "e4m3" else TOL[wl.act]
