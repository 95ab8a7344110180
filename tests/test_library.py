"""Host-side checks of the C-ABI library (no GPU, no kernel launches).

The library must load, export every entry point that include/moe.h declares,
size its workspace, and reject bad arguments on the host before touching the
GPU (every call here fails validation, so nothing is launched).
"""

import ctypes
import os
import re

import pytest
import torch

import sparse_moe_ffn_route_amd as moe
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_symbol():
    lib = moe.library()
    names = declared_functions()
    assert set(names) == set(moe.EXPORTS)
    for name in names:
        assert hasattr(lib, name), name
    assert lib.moe_abi_version() == 4


def test_library_targets_gfx950_only():
    blob = open(moe.LIB_PATH, "rb").read()
    assert b"gfx950" in blob
    for other in (b"gfx942", b"gfx90a", b"gfx1100"):
        assert other not in blob


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_workspace_bytes_for_every_workload(name):
    wl = synth.WORKLOADS[name]
    n = moe.moe_workspace_bytes(moe.make_dims(wl.T, wl.D, wl.E, wl.top_k, wl.I, wl.I_shared, wl.expert_begin,
                                              wl.local, True, wl.act, wl.w, wl.out))
    tk = wl.T * wl.top_k
    out_b = 4 if wl.out == "f32" else 2
    assert n >= tk * wl.D * out_b          # at least the grouped expert outputs
    assert n % 256 == 0
    assert n < 4 * 2 ** 30


def _dims(**kw):
    base = dict(T=8, D=64, E=8, top_k=2, I=64, I_shared=0, expert_begin=0, n_local=None, renormalize=True,
                act="bf16", w="bf16", out="bf16")
    base.update(kw)
    return moe.make_dims(**base)


BAD_DIMS = [dict(T=-1), dict(D=0), dict(E=0), dict(top_k=0), dict(top_k=9), dict(I=0), dict(I_shared=-64),
            dict(expert_begin=6, n_local=4), dict(expert_begin=-1, n_local=2)]


def test_pack_weights_argument_checks():
    lib = moe.library()
    fake = ctypes.c_void_p(256)
    assert lib.moe_pack_weights(3, 1, 16, 64, fake, fake, None) == moe.ERR_UNSUPPORTED      # dtype
    assert lib.moe_pack_weights(moe.BF16, 1, 24, 64, fake, fake, None) == moe.ERR_UNSUPPORTED  # rows % 16
    assert lib.moe_pack_weights(moe.BF16, 1, 16, 48, fake, fake, None) == moe.ERR_UNSUPPORTED  # 96 B rows
    assert lib.moe_pack_weights(moe.BF16, -1, 16, 64, fake, fake, None) == moe.ERR_BAD_DIMS
    assert lib.moe_pack_weights(moe.BF16, 1, 16, 64, None, fake, None) == moe.ERR_NULL_ARG
    assert lib.moe_pack_weights(moe.BF16, 0, 16, 64, None, None, None) == moe.OK              # nothing to do


def test_hbm_read_probe_argument_checks():
    lib = moe.library()
    fake = ctypes.c_void_p(256)
    assert lib.moe_hbm_read_probe(fake, 24, fake, None) == moe.ERR_UNSUPPORTED   # not whole 16-byte chunks
    assert lib.moe_hbm_read_probe(None, 32, fake, None) == moe.ERR_NULL_ARG
    assert lib.moe_hbm_read_probe(fake, 32, None, None) == moe.ERR_NULL_ARG
    assert lib.moe_hbm_read_probe(None, 0, None, None) == moe.OK                  # nothing to read


def test_mfma_peak_probe_argument_checks():
    lib = moe.library()
    fake = ctypes.c_void_p(256)
    assert lib.moe_mfma_peak_probe(moe.F32, 10, fake, None) == moe.ERR_UNSUPPORTED
    assert lib.moe_mfma_peak_probe(moe.BF16, 0, fake, None) == moe.ERR_BAD_DIMS
    assert lib.moe_mfma_peak_probe(moe.E4M3, 10, None, None) == moe.ERR_NULL_ARG


UNSUPPORTED = [dict(D=96), dict(I=100), dict(I_shared=32), dict(E=2048, top_k=2), dict(E=64, top_k=33),
               dict(act="f32", w="bf16"), dict(act="f32", w="f32", out="bf16"), dict(act="bf16", w="f32"),
               dict(act="e4m3", w="e4m3"),
               # one expert's weight matrix (I x D) or the router's (E x D) of 2 GiB or more
               dict(D=65536, I=16384, I_shared=0), dict(D=1 << 20, E=1024, I=64, I_shared=0)]


@pytest.mark.parametrize("kw", BAD_DIMS)
def test_bad_dims_rejected(kw):
    assert moe.moe_workspace_bytes(_dims(**kw)) == 0
    lib = moe.library()
    fake = ctypes.c_void_p(256)
    st = lib.moe_route(ctypes.byref(_dims(**kw)), None, None, fake, None, fake, None, 0, None)
    assert st == moe.ERR_BAD_DIMS


@pytest.mark.parametrize("kw", UNSUPPORTED)
def test_unsupported_rejected(kw):
    assert moe.moe_workspace_bytes(_dims(**kw)) == 0
    lib = moe.library()
    fake = ctypes.c_void_p(256)
    st = lib.moe_route(ctypes.byref(_dims(**kw)), None, None, fake, None, fake, None, 0, None)
    assert st == moe.ERR_UNSUPPORTED


def test_null_arguments_rejected():
    lib = moe.library()
    d = _dims()
    fake = ctypes.c_void_p(256)
    assert lib.moe_workspace_bytes(None) == 0
    assert lib.moe_route(None, None, None, fake, None, fake, None, 0, None) == moe.ERR_NULL_ARG
    assert lib.moe_route(ctypes.byref(d), None, None, None, None, fake, None, 0, None) == moe.ERR_NULL_ARG
    # x without a router weight
    assert lib.moe_route(ctypes.byref(d), fake, None, fake, None, fake, None, 0, None) == moe.ERR_NULL_ARG
    assert lib.moe_permute(ctypes.byref(d), None, fake, fake, fake, fake, None, None, None, fake, 1 << 20,
                           None) == moe.ERR_NULL_ARG
    assert lib.moe_unpermute_combine(ctypes.byref(d), fake, fake, None, None, fake, None) == moe.ERR_NULL_ARG
    w = moe.moe_weights(None, fake, fake, fake, None, None, None, None, None, None)
    # neither a router weight nor a given routing
    assert lib.moe_layer_forward(ctypes.byref(d), ctypes.byref(w), fake, None, None, fake, None, None, fake,
                                 1 << 30, None, None) == moe.ERR_NULL_ARG
    # fp8 weights without scales
    d8 = _dims(w="e4m3")
    assert lib.moe_grouped_ffn(ctypes.byref(d8), fake, fake, None, fake, fake, fake, fake, None, None, None, fake,
                               fake, 1 << 30, None) == moe.ERR_NULL_ARG


def test_small_workspace_rejected():
    lib = moe.library()
    d = _dims()
    need = moe.moe_workspace_bytes(d)
    fake = ctypes.c_void_p(256)
    st = lib.moe_permute(ctypes.byref(d), fake, fake, fake, fake, fake, None, None, None, fake, need - 1, None)
    assert st == moe.ERR_WORKSPACE
    w = moe.moe_weights(fake, fake, fake, fake, None, None, None, None, None, None)
    st = lib.moe_layer_forward(ctypes.byref(d), ctypes.byref(w), fake, None, None, fake, None, None, fake, need - 1,
                               None, None)
    assert st == moe.ERR_WORKSPACE


def test_zero_tokens_is_a_no_op():
    lib = moe.library()
    d = _dims(T=0)
    need = moe.moe_workspace_bytes(d)
    fake = ctypes.c_void_p(256)
    w = moe.moe_weights(fake, fake, fake, fake, None, None, None, None, None, None)
    assert lib.moe_layer_forward(ctypes.byref(d), ctypes.byref(w), fake, None, None, fake, None, None, fake, need,
                                 None, None) == moe.OK
    assert lib.moe_route(ctypes.byref(d), None, None, fake, None, fake, None, 0, None) == moe.OK


def test_status_strings():
    lib = moe.library()
    for code in (0, -1, -2, -3, -4, -5):
        assert lib.moe_status_string(code)
    assert lib.moe_last_hip_error() == 0


def test_binding_refuses_tensors_smaller_than_the_dims():
    """The kernels trust the dims: a hidden-state tensor with fewer rows than T must be refused before
    any launch (a 32768-token layer handed 8192 rows would read past the end of x)."""
    d = moe.make_dims(32768, 256, 16, 2, 64)
    x_short = torch.zeros(8192, 256, dtype=torch.bfloat16)
    y = torch.zeros(32768, 256, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="x:"):
        moe.moe_layer_forward(d, moe.make_weights(), x_short, None, None, y)
    with pytest.raises(ValueError, match="logits"):
        moe.moe_route(d, None, None, torch.zeros(10, dtype=torch.float32), None,
                      torch.zeros(32768 * 4, dtype=torch.int32))
    with pytest.raises(ValueError, match="perm_token"):
        moe.moe_permute(d, torch.zeros(32768 * 4, dtype=torch.int32), torch.zeros(16, dtype=torch.int32),
                        torch.zeros(17, dtype=torch.int32), torch.zeros(5, dtype=torch.int32),
                        torch.zeros(32768 * 2, dtype=torch.int32))


def test_fused_router_argument_checks():
    lib = moe.library()
    fake = ctypes.c_void_p(256)
    big_x = moe.make_dims(65536, 16384, 16, 4, 64)              # x of 2 GiB: past the 32-bit offsets
    n = moe.moe_workspace_bytes(big_x)
    assert lib.moe_route_fused(ctypes.byref(big_x), fake, fake, None, None, fake, fake, n, None) == moe.ERR_UNSUPPORTED
    d = moe.make_dims(64, 256, 16, 4, 64)
    n = moe.moe_workspace_bytes(d)
    assert lib.moe_route_fused(ctypes.byref(d), None, fake, None, None, fake, fake, n, None) == moe.ERR_NULL_ARG
    assert lib.moe_route_fused(ctypes.byref(d), fake, fake, None, None, None, fake, n, None) == moe.ERR_NULL_ARG
    assert lib.moe_route_fused(ctypes.byref(d), fake, fake, None, None, fake, None, n, None) == moe.ERR_NULL_ARG
    assert lib.moe_route_fused(ctypes.byref(d), fake, fake, None, None, fake, fake, n - 1, None) == moe.ERR_WORKSPACE
    zero = moe.make_dims(0, 256, 16, 4, 64)
    assert lib.moe_route_fused(ctypes.byref(zero), fake, fake, None, None, fake, fake, 1 << 20, None) == moe.OK


def test_audit_argument_checks():
    lib = moe.library()
    fake = ctypes.c_void_p(256)
    d = moe.make_dims(64, 256, 16, 4, 64, 64)
    assert lib.moe_audit_workspace_bytes(ctypes.byref(d), 0) == 0
    assert lib.moe_audit_workspace_bytes(ctypes.byref(d), 5000) == 0
    assert lib.moe_audit_workspace_bytes(ctypes.byref(d), 16) > 16 * 5 * (256 + 64) * 4
    w = moe.moe_weights(fake, fake, fake, fake, None, None, None, fake, fake, fake)
    n = lib.moe_audit_workspace_bytes(ctypes.byref(d), 4)
    assert lib.moe_audit(ctypes.byref(d), ctypes.byref(w), None, fake, fake, fake, 4, None, fake, fake, n,
                         None) == moe.ERR_NULL_ARG
    assert lib.moe_audit(ctypes.byref(d), ctypes.byref(w), fake, fake, fake, fake, 4, None, fake, fake, n - 1,
                         None) == moe.ERR_WORKSPACE
    assert lib.moe_audit(ctypes.byref(d), ctypes.byref(w), fake, fake, fake, fake, 0, None, fake, fake, n,
                         None) == moe.ERR_BAD_DIMS
    wide = moe.make_dims(64, 32768, 16, 4, 64)
    assert lib.moe_audit(ctypes.byref(wide), ctypes.byref(w), fake, fake, fake, fake, 4, None, fake, fake, 1 << 30,
                         None) == moe.ERR_UNSUPPORTED
    fp8 = moe.make_dims(64, 256, 16, 4, 64, w="e4m3")
    assert lib.moe_audit(ctypes.byref(fp8), ctypes.byref(w), fake, fake, fake, fake, 4, None, fake, fake, 1 << 30,
                         None) == moe.ERR_NULL_ARG                              # scales missing
