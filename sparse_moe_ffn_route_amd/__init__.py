"""Routed Mixture-of-Experts FFN layer for AMD MI355X (gfx950).

Thin ctypes binding over ``libmoe_hip.so`` (C ABI in ``include/moe.h``).  The
functions below carry the C names and only marshal arguments: torch tensors
become device pointers, the current torch stream becomes the HIP stream.
Every step of the layer runs in the library's HIP kernels; there is no
fallback.  Loading fails loudly when the library has not been built
(``python -m sparse_moe_ffn_route_amd.build``).
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_hip.so")

# enum moe_dtype
F32, BF16, E4M3 = 0, 1, 2
_DTYPE_CODE = {"f32": F32, "bf16": BF16, "e4m3": E4M3}
_TORCH_OF = {F32: torch.float32, BF16: torch.bfloat16, E4M3: torch.float8_e4m3fn}

# enum moe_layout
LAYOUT_ROWS, LAYOUT_PACKED = 0, 1
_LAYOUT_CODE = {"rows": LAYOUT_ROWS, "packed": LAYOUT_PACKED}

# enum moe_status
OK, ERR_NULL_ARG, ERR_BAD_DIMS, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP, ERR_SCRATCH_LIMIT = 0, -1, -2, -3, -4, -5, -6

WS_ERROR_OFFSET = 0                     # MOE_WS_ERROR_OFFSET: byte offset of the workspace error word
STATIC_SCRATCH_BYTES = 96 << 20         # MOE_STATIC_SCRATCH_BYTES

# Symbols exported by the library (the entry points of include/moe.h).
EXPORTS = (
    "moe_workspace_bytes", "moe_route", "moe_route_fused", "moe_permute", "moe_grouped_ffn",
    "moe_unpermute_combine", "moe_layer_forward", "moe_layer_forward_noalloc", "moe_audit_workspace_bytes", "moe_audit", "moe_pack_weights", "moe_hbm_read_probe", "moe_status_string", "moe_last_hip_error",
    "moe_abi_version", "moe_mfma_peak_probe",
)


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: status {status}")
        self.status = status


class moe_dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "T", "D", "E", "top_k", "I", "I_shared", "expert_begin", "n_local", "renormalize",
        "act_dtype", "w_dtype", "out_dtype", "weight_layout")]


class moe_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "w_router", "w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down", "sh_gate", "sh_up", "sh_down")]


_lib = None


ABI_VERSION = 4   # moe_abi_version() of the library these signatures describe


def library() -> ctypes.CDLL:
    """Load ``libmoe_hip.so`` (raises if it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m sparse_moe_ffn_route_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    dp, wp = ctypes.POINTER(moe_dims), ctypes.POINTER(moe_weights)
    lib.moe_workspace_bytes.argtypes = [dp]
    lib.moe_workspace_bytes.restype = sz
    lib.moe_route.argtypes = [dp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_route.restype = i32
    lib.moe_route_fused.argtypes = [dp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_route_fused.restype = i32
    lib.moe_permute.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_permute.restype = i32
    lib.moe_grouped_ffn.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_grouped_ffn.restype = i32
    lib.moe_unpermute_combine.argtypes = [dp, vp, vp, vp, vp, vp, vp]
    lib.moe_unpermute_combine.restype = i32
    lib.moe_layer_forward.argtypes = [dp, wp, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp]
    lib.moe_layer_forward.restype = i32
    lib.moe_layer_forward_noalloc.argtypes = [dp, wp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.moe_layer_forward_noalloc.restype = i32
    lib.moe_pack_weights.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, vp, vp, vp]
    lib.moe_pack_weights.restype = i32
    lib.moe_audit_workspace_bytes.argtypes = [dp, ctypes.c_int32]
    lib.moe_audit_workspace_bytes.restype = sz
    lib.moe_audit.argtypes = [dp, wp, vp, vp, vp, vp, ctypes.c_int32, vp, vp, vp, sz, vp]
    lib.moe_audit.restype = i32
    lib.moe_hbm_read_probe.argtypes = [vp, sz, vp, vp]
    lib.moe_hbm_read_probe.restype = i32
    lib.moe_mfma_peak_probe.argtypes = [ctypes.c_int32, ctypes.c_int32, vp, vp]
    lib.moe_mfma_peak_probe.restype = i32
    lib.moe_status_string.argtypes = [i32]
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_last_hip_error.argtypes = []
    lib.moe_last_hip_error.restype = i32
    lib.moe_abi_version.argtypes = []
    lib.moe_abi_version.restype = i32
    if lib.moe_abi_version() != ABI_VERSION:
        raise ImportError(f"{LIB_PATH} has ABI version {lib.moe_abi_version()}, this binding expects {ABI_VERSION}: "
                          "rebuild it with `python -m sparse_moe_ffn_route_amd.build`")
    _lib = lib
    return lib


def make_dims(T, D, E, top_k, I, I_shared=0, expert_begin=0, n_local=None, renormalize=True,
              act="bf16", w="bf16", out="bf16", layout="rows") -> moe_dims:
    return moe_dims(T, D, E, top_k, I, I_shared, expert_begin, E if n_local is None else n_local,
                    1 if renormalize else 0, _DTYPE_CODE[act], _DTYPE_CODE[w], _DTYPE_CODE[out],
                    _LAYOUT_CODE[layout])


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor or None")
    if t.device.type != "cuda":
        raise ValueError("tensors must live in GPU memory")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status: int, what: str):
    if status != OK:
        lib = library()
        msg = lib.moe_status_string(status).decode()
        if status == ERR_HIP:
            msg += f" (hipError {lib.moe_last_hip_error()})"
        raise MoeError(status, f"{what}: {msg}")


def moe_workspace_bytes(dims: moe_dims) -> int:
    return int(library().moe_workspace_bytes(ctypes.byref(dims)))


def workspace(dims: moe_dims, device="cuda") -> torch.Tensor:
    """A caller-owned scratch buffer of moe_workspace_bytes(dims) bytes."""
    n = moe_workspace_bytes(dims)
    if n == 0:
        raise MoeError(ERR_BAD_DIMS, "moe_workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=device)


_ELEM_BYTES = {F32: 4, BF16: 2, E4M3: 1}


def _need(t: Optional[torch.Tensor], nbytes: int, what: str):
    """Refuse a tensor smaller than the dims say (the kernels trust the dims)."""
    if t is not None and t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{what}: {t.numel() * t.element_size()} bytes, the dims need {nbytes}")


def _check_io(dims, x=None, logits=None, packed=None, bias=None, y=None, w_router=None):
    T, D, E, k = dims.T, dims.D, dims.E, dims.top_k
    _need(x, T * D * _ELEM_BYTES[dims.act_dtype], "x")
    _need(w_router, E * D * _ELEM_BYTES[dims.act_dtype], "w_router")
    _need(logits, T * E * 4, "logits")
    _need(packed, T * 2 * k * 4, "packed routing")
    _need(bias, E * 4, "logit bias")
    _need(y, T * D * _ELEM_BYTES[dims.out_dtype], "y")


def moe_route(dims, x, w_router, logits, logit_bias, packed, ws=None, stream=None):
    _check_io(dims, x=x, logits=logits, packed=packed, bias=logit_bias, w_router=w_router)
    _check(library().moe_route(ctypes.byref(dims), _ptr(x), _ptr(w_router), _ptr(logits), _ptr(logit_bias),
                               _ptr(packed), _ptr(ws), ws.numel() if ws is not None else 0, _stream(stream)),
           "moe_route")


def moe_route_fused(dims, x, w_router, logits, logit_bias, packed, ws=None, stream=None):
    """Fused projection + top-k + blob (logits: optional fp32 copy, or None)."""
    _check_io(dims, x=x, logits=logits, packed=packed, bias=logit_bias, w_router=w_router)
    if ws is None:
        ws = workspace(dims, device=x.device)
    _check(library().moe_route_fused(ctypes.byref(dims), _ptr(x), _ptr(w_router), _ptr(logits), _ptr(logit_bias),
                                     _ptr(packed), _ptr(ws), ws.numel(), _stream(stream)), "moe_route_fused")


def moe_permute(dims, packed, counts, offsets, perm_token, inv_pos, x=None, x_perm=None, x_perm_scale=None,
                ws=None, stream=None):
    tk = dims.T * dims.top_k
    _check_io(dims, x=x, packed=packed)
    _need(counts, dims.n_local * 4, "counts")
    _need(offsets, (dims.n_local + 1) * 4, "offsets")
    _need(perm_token, tk * 4, "perm_token")
    _need(inv_pos, tk * 4, "inv_pos")
    _need(x_perm, tk * dims.D * (1 if dims.w_dtype == E4M3 else _ELEM_BYTES[dims.act_dtype]), "x_perm")
    _check(library().moe_permute(ctypes.byref(dims), _ptr(packed), _ptr(counts), _ptr(offsets), _ptr(perm_token),
                                 _ptr(inv_pos), _ptr(x), _ptr(x_perm), _ptr(x_perm_scale), _ptr(ws),
                                 ws.numel() if ws is not None else 0, _stream(stream)), "moe_permute")


def moe_grouped_ffn(dims, a_rows, a_scale, perm_token, offsets, w_gate, w_up, w_down, s_gate, s_up, s_down,
                    out_rows, ws, stream=None):
    _check(library().moe_grouped_ffn(ctypes.byref(dims), _ptr(a_rows), _ptr(a_scale), _ptr(perm_token),
                                     _ptr(offsets), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(s_gate),
                                     _ptr(s_up), _ptr(s_down), _ptr(out_rows), _ptr(ws),
                                     ws.numel() if ws is not None else 0, _stream(stream)), "moe_grouped_ffn")


def moe_unpermute_combine(dims, out_rows, packed, inv_pos, shared_out, y, stream=None):
    _check_io(dims, packed=packed, y=y)
    _need(inv_pos, dims.T * dims.top_k * 4, "inv_pos")
    _need(shared_out, dims.T * dims.D * _ELEM_BYTES[dims.out_dtype], "shared_out")
    _check(library().moe_unpermute_combine(ctypes.byref(dims), _ptr(out_rows), _ptr(packed), _ptr(inv_pos),
                                           _ptr(shared_out), _ptr(y), _stream(stream)), "moe_unpermute_combine")


def make_weights(w_router=None, w_gate=None, w_up=None, w_down=None, s_gate=None, s_up=None, s_down=None,
                 sh_gate=None, sh_up=None, sh_down=None) -> moe_weights:
    """moe_weights from tensors; the tensors must stay alive while the struct is used."""
    return moe_weights(*[_ptr(t) for t in (w_router, w_gate, w_up, w_down, s_gate, s_up, s_down,
                                           sh_gate, sh_up, sh_down)])


STAGE_EVENTS = 7   # MOE_STAGE_EVENTS
STAGES = ("route", "permute", "gate_up", "down", "shared", "combine")


def moe_layer_forward(dims, weights: moe_weights, x, packed_in, logit_bias, y, logits_out=None, packed_out=None,
                      ws=None, stage_events=None, stream=None):
    """stage_events: None or STAGE_EVENTS recorded torch.cuda.Event(enable_timing=True) objects."""
    ev = None
    if stage_events is not None:
        if len(stage_events) != STAGE_EVENTS:
            raise ValueError(f"stage_events needs {STAGE_EVENTS} events")
        for e in stage_events:
            if not e.cuda_event:
                e.record()   # torch creates the underlying hipEvent on its first record
        ev = (ctypes.c_void_p * STAGE_EVENTS)(*[e.cuda_event for e in stage_events])
    _check_io(dims, x=x, logits=logits_out, packed=packed_in, bias=logit_bias, y=y)
    _need(packed_out, dims.T * 2 * dims.top_k * 4, "packed_out")
    _check(library().moe_layer_forward(ctypes.byref(dims), ctypes.byref(weights), _ptr(x), _ptr(packed_in),
                                       _ptr(logit_bias), _ptr(y), _ptr(logits_out), _ptr(packed_out), _ptr(ws),
                                       ws.numel() if ws is not None else 0, ev, _stream(stream)),
           "moe_layer_forward")


def moe_layer_forward_noalloc(dims, weights: moe_weights, x, packed_in, logit_bias, y, logits_out=None,
                              packed_out=None, bad_ids=None, stage_events=None, stream=None):
    """moe_layer_forward on the library's static device scratch (no workspace argument).

    bad_ids: None or a device int32 tensor that receives the count of routing-blob ids outside [0, E).
    """
    ev = None
    if stage_events is not None:
        if len(stage_events) != STAGE_EVENTS:
            raise ValueError(f"stage_events needs {STAGE_EVENTS} events")
        for e in stage_events:
            if not e.cuda_event:
                e.record()
        ev = (ctypes.c_void_p * STAGE_EVENTS)(*[e.cuda_event for e in stage_events])
    _check_io(dims, x=x, logits=logits_out, packed=packed_in, bias=logit_bias, y=y)
    _need(packed_out, dims.T * 2 * dims.top_k * 4, "packed_out")
    _need(bad_ids, 4, "bad_ids")
    _check(library().moe_layer_forward_noalloc(ctypes.byref(dims), ctypes.byref(weights), _ptr(x), _ptr(packed_in),
                                               _ptr(logit_bias), _ptr(y), _ptr(logits_out), _ptr(packed_out),
                                               _ptr(bad_ids), ev, _stream(stream)),
           "moe_layer_forward_noalloc")


def workspace_error_count(ws: torch.Tensor) -> torch.Tensor:
    """View of the workspace error word (ids outside [0, E) seen by the last grouping on ws), as int32 [1]."""
    return ws[WS_ERROR_OFFSET:WS_ERROR_OFFSET + 4].view(torch.int32)


def moe_audit(dims, weights: moe_weights, x, packed, y, sample, ref_out=None, stream=None):
    """fp32 shadow of the layer on the sampled tokens; returns a device tensor [max |y - ref|, max |ref|]."""
    n = sample.numel()
    _check_io(dims, x=x, packed=packed, y=y)
    _need(ref_out, n * dims.D * 4, "ref_out")
    nbytes = int(library().moe_audit_workspace_bytes(ctypes.byref(dims), n))
    if nbytes == 0:
        raise MoeError(ERR_BAD_DIMS, "moe_audit_workspace_bytes")
    ws = torch.empty(nbytes, dtype=torch.uint8, device=x.device)
    result = torch.empty(2, dtype=torch.float32, device=x.device)
    _check(library().moe_audit(ctypes.byref(dims), ctypes.byref(weights), _ptr(x), _ptr(packed), _ptr(y),
                               _ptr(sample), n, _ptr(ref_out), _ptr(result), _ptr(ws), nbytes, _stream(stream)),
           "moe_audit")
    return result


_CODE_OF_TORCH = {torch.float32: F32, torch.bfloat16: BF16, torch.float8_e4m3fn: E4M3, torch.uint8: E4M3}


def moe_pack_weights(src: torch.Tensor, dst: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Repack [n][rows][cols] (or [rows][cols]) row-major weights into the fragment-major layout."""
    if src.dim() == 2:
        n, rows, cols = 1, src.shape[0], src.shape[1]
    elif src.dim() == 3:
        n, rows, cols = src.shape
    else:
        raise ValueError("weights must be [rows][cols] or [n][rows][cols]")
    if dst is None:
        dst = torch.empty_like(src)
    if dst.shape != src.shape or dst.dtype != src.dtype:
        raise ValueError("dst must match src in shape and dtype")
    _check(library().moe_pack_weights(_CODE_OF_TORCH[src.dtype], n, rows, cols, _ptr(src), _ptr(dst),
                                      _stream(stream)), "moe_pack_weights")
    return dst


HBM_PROBE_SINK_WORDS = 16384


def moe_hbm_read_probe(buf: torch.Tensor, sink: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Read all of buf once (measurement helper); returns the checksum words."""
    nbytes = buf.numel() * buf.element_size()
    if sink is None:
        sink = torch.empty(HBM_PROBE_SINK_WORDS, dtype=torch.int32, device=buf.device)
    if sink.numel() * sink.element_size() < HBM_PROBE_SINK_WORDS * 4:
        raise ValueError("sink must hold 16384 32-bit words")
    _check(library().moe_hbm_read_probe(_ptr(buf), nbytes - nbytes % 16, _ptr(sink), _stream(stream)),
           "moe_hbm_read_probe")
    return sink


MFMA_PROBE_BLOCKS = 2048   # MOE_MFMA_PROBE_BLOCKS
_MFMA_PROBE_FLOP = {BF16: 16384, E4M3: 65536}


def moe_mfma_peak_probe(dtype: str, iters: int, sink: Optional[torch.Tensor] = None, stream=None):
    """Launch the MFMA throughput probe; returns (sink tensor, FLOP of the launch)."""
    code = _DTYPE_CODE[dtype]
    if sink is None:
        sink = torch.empty(MFMA_PROBE_BLOCKS, dtype=torch.float32, device="cuda")
    _need(sink, MFMA_PROBE_BLOCKS * 4, "sink")
    _check(library().moe_mfma_peak_probe(code, iters, _ptr(sink), _stream(stream)), "moe_mfma_peak_probe")
    return sink, MFMA_PROBE_BLOCKS * 4 * 8 * iters * _MFMA_PROBE_FLOP.get(code, 0)


def torch_dtype(code: int) -> torch.dtype:
    return _TORCH_OF[code]
