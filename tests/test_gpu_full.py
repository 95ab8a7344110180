"""GPU parity at the full workload sizes, in the launch configuration the bench times.

Every token's routing is checked bit-exactly (ids) against the oracle fed the
GPU's fp32 logits, the grouping of all T*k pairs bit-exactly, the router logits
on sampled tokens against the fp32 accumulation bound, and y on sampled tokens
(the oracle evaluates only those tokens' experts; every row of the layer is
independent, so this is exactly the oracle's value for those tokens).
"""

import numpy as np
import pytest
import torch

import oracle
import sparse_moe_ffn_route_amd as moe
import synth
from harness import dims_of, gpu_layer, logit_bound, rel_err, tolerance

pytestmark = pytest.mark.gpu

SAMPLE = 12


@pytest.fixture(scope="module")
def big_layer():
    """Weights of the D=4096, E=512, I=1024 layer (12.9 GB bf16), drawn once on the GPU."""
    inp = synth.make_inputs(synth.WORKLOADS["prefill_bf16"], 0, "cuda")
    yield inp
    del inp
    torch.cuda.empty_cache()


def _variant(big, name):
    wl = synth.WORKLOADS[name]
    x = big.x[: wl.T].contiguous()
    bias = None
    if wl.skew_alpha is not None:
        bias = torch.from_numpy(synth.zipf_bias(wl.E, wl.skew_alpha, wl.skew_s, wl.skew_empty, 1)).cuda()
    return synth.LayerInputs(wl, x, big.w_router, big.w_gate, big.w_up, big.w_down, None, None, None,
                             big.ws_gate, big.ws_up, big.ws_down, bias, None)


def _sample_tokens(T, seed):
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(T, size=min(SAMPLE, T), replace=False))


def _check_grouping(inp, packed_np):
    wl = inp.wl
    d = dims_of(wl)
    T, k = wl.T, wl.top_k
    counts = torch.empty(wl.local, dtype=torch.int32, device="cuda")
    offsets = torch.empty(wl.local + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(T * k, dtype=torch.int32, device="cuda")
    inv = torch.empty(T, k, dtype=torch.int32, device="cuda")
    moe.moe_permute(d, torch.from_numpy(packed_np).cuda(), counts, offsets, perm, inv, ws=moe.workspace(d))
    ids, _ = oracle.unpack_routing(packed_np)
    c, o, p, iv = oracle.permute(ids, wl.expert_begin, wl.local)
    np.testing.assert_array_equal(counts.cpu().numpy(), c)
    np.testing.assert_array_equal(offsets.cpu().numpy(), o)
    np.testing.assert_array_equal(perm.cpu().numpy()[: int(o[-1])], p)
    np.testing.assert_array_equal(inv.cpu().numpy(), iv)
    return c


def _check_routed_layer(inp, seed, packed=True):
    wl = inp.wl
    g = gpu_layer(inp, packed=packed)
    # routing of every token, from the GPU's fp32 logits
    bias = None if inp.bias is None else inp.bias.cpu().numpy()
    ids, w = oracle.route(g["logits"], wl.top_k, bias=bias, renormalize=wl.renormalize)
    ids_gpu, w_gpu = oracle.unpack_routing(g["packed"])
    np.testing.assert_array_equal(ids_gpu, ids)
    np.testing.assert_allclose(w_gpu, w, rtol=0, atol=1e-6)
    counts = _check_grouping(inp, g["packed"])
    s = _sample_tokens(wl.T, seed)
    x_s = synth.f64(inp.x[torch.from_numpy(s).cuda()])
    wr = synth.f64(inp.w_router)
    l_ref = oracle.router_logits(x_s, wr).astype(np.float64)
    assert np.all(np.abs(g["logits"][s] - l_ref) <= logit_bound(x_s, wr, l_ref))
    ref = oracle.layer_from_routing(x_s, ids[s], w[s], synth.ExpertView(inp), shared=synth.shared_f64(inp))
    err = rel_err(g["y"][s], ref["y"])
    assert err <= tolerance(wl), f"{wl.name}: sampled rel err {err:.3e}"
    # the routed part alone (shared expert off) on the same tokens, row-major weights
    g2 = gpu_layer(inp, shared=False, packed=False)
    ref2 = oracle.layer_from_routing(x_s, ids[s], w[s], synth.ExpertView(inp), shared=None)
    err2 = rel_err(g2["y"][s], ref2["y"])
    assert err2 <= tolerance(wl), f"{wl.name} (no shared): sampled rel err {err2:.3e}"
    return counts


def test_decode_full_size(big_layer):
    counts = _check_routed_layer(_variant(big_layer, "decode_bf16"), 10)
    assert counts.sum() == 512 * 10


def test_prefill_full_size(big_layer):
    counts = _check_routed_layer(_variant(big_layer, "prefill_bf16"), 11)
    assert counts.sum() == 8192 * 10


def test_prefill32k_full_size(big_layer):
    """The 32K-token probe: experts of ~640 rows span three 256-row M-tiles."""
    wl = synth.WORKLOADS["prefill32k_bf16"]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(32768)
    x = torch.randn(wl.T, wl.D, generator=gen, device="cuda").to(torch.bfloat16)
    b = big_layer
    inp = synth.LayerInputs(wl, x, b.w_router, b.w_gate, b.w_up, b.w_down, None, None, None, b.ws_gate, b.ws_up,
                            b.ws_down, None, None)
    counts = _check_routed_layer(inp, 15)
    assert counts.sum() == 32768 * 10 and counts.min() > 256


def test_skewed_prefill_full_size(big_layer):
    counts = _check_routed_layer(_variant(big_layer, "skew_prefill_bf16"), 12)
    assert (counts == 0).sum() == 32                      # the never-chosen experts stay empty
    assert counts.max() / counts.mean() > 15              # a straggler expert many times the mean load


def test_ep_share_fp8_full_size():
    wl = synth.WORKLOADS["ep_share_fp8"]
    inp = synth.make_inputs(wl, 0, "cuda")
    g = gpu_layer(inp, packed=True)
    np.testing.assert_array_equal(g["packed"], inp.packed.cpu().numpy())   # the given blob passes through
    counts = _check_grouping(inp, g["packed"])
    assert 9000 < counts.sum() < 11500                    # ~T*k*64/512 pairs are local
    ids, w32 = oracle.unpack_routing(inp.packed.cpu().numpy())
    local_tok = np.nonzero(((ids >= 0) & (ids < 64)).any(axis=1))[0]
    s = np.sort(np.random.default_rng(13).choice(local_tok, size=SAMPLE, replace=False))
    x_s = synth.f64(inp.x[torch.from_numpy(s).cuda()])
    ref = oracle.layer_from_routing_fp8(x_s, ids[s], w32[s].astype(np.float64), synth.ExpertViewFP8(inp),
                                        expert_begin=0, n_local=64)
    err = rel_err(g["y"][s], ref["y"])
    assert err <= tolerance(wl), f"fp8 share: sampled rel err {err:.3e}"
    # tokens with no local expert get an all-zero partial sum
    none_local = np.nonzero(~((ids >= 0) & (ids < 64)).any(axis=1))[0]
    assert none_local.size > 0 and np.all(g["y"][none_local] == 0)


def test_decode_fp8_full_size():
    """The decode batch with e4m3 routed experts (router and shared expert bf16)."""
    wl = synth.WORKLOADS["decode_fp8"]
    inp = synth.make_inputs(wl, 0, "cuda")
    g = gpu_layer(inp, packed=True)
    ids, w = oracle.route(g["logits"], wl.top_k, renormalize=wl.renormalize)
    ids_gpu, w_gpu = oracle.unpack_routing(g["packed"])
    np.testing.assert_array_equal(ids_gpu, ids)
    np.testing.assert_allclose(w_gpu, w, rtol=0, atol=1e-6)
    counts = _check_grouping(inp, g["packed"])
    assert counts.sum() == 512 * 10
    s = _sample_tokens(wl.T, 14)
    x_s = synth.f64(inp.x[torch.from_numpy(s).cuda()])
    wr = synth.f64(inp.w_router)
    l_ref = oracle.router_logits(x_s, wr).astype(np.float64)
    assert np.all(np.abs(g["logits"][s] - l_ref) <= logit_bound(x_s, wr, l_ref))
    ref = oracle.layer_from_routing_fp8(x_s, ids[s], w[s], synth.ExpertViewFP8(inp), shared=synth.shared_f64(inp))
    err = rel_err(g["y"][s], ref["y"])
    assert err <= tolerance(wl), f"decode fp8: sampled rel err {err:.3e}"
    del inp
    torch.cuda.empty_cache()


def test_operands_past_2gib_take_the_streaming_shape():
    """65536 tokens x top-8 x I = 1024 puts the grouped h rows past 2 GiB (fp32 bound): the
    grouped GEMMs fall back from the 256-row tile shape to the 32-row streaming shape."""
    wl = synth.Workload("big_rows", T=65536, D=256, E=64, top_k=8, I=1024, I_shared=0, act="bf16", w="bf16",
                        out="bf16")
    inp = synth.make_inputs(wl, 0, "cuda")
    g = gpu_layer(inp, packed=True)
    ids, w = oracle.route(g["logits"], wl.top_k)
    np.testing.assert_array_equal(oracle.unpack_routing(g["packed"])[0], ids)
    s = _sample_tokens(wl.T, 16)
    x_s = synth.f64(inp.x[torch.from_numpy(s).cuda()])
    ref = oracle.layer_from_routing(x_s, ids[s], w[s], synth.ExpertView(inp))
    err = rel_err(g["y"][s], ref["y"])
    assert err <= tolerance(wl), f"past-2GiB batch: sampled rel err {err:.3e}"
    del inp
    torch.cuda.empty_cache()
