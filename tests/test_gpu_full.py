"""GPU parity at the full workload sizes, in the launch configuration the bench times.

Every token's routing is checked bit-exactly (ids) against the oracle fed the
GPU's fp32 logits, the grouping of all T*k pairs bit-exactly, the router logits
on sampled tokens against the fp32 accumulation bound, and y on EVERY token of
the 512-token decode batches, the 8192-token prefill chunks and the fp8
expert-parallel share, with and without the shared expert (the shared expert
dominates y, so a routed-path error could hide under the tolerance with it on).
The 32K-token probe checks y on tokens chosen to reach the grouped GEMMs' corner
cases (the ragged last M-tile of the largest experts, rows 192-255 of 256-row
tiles) plus random ones; every row of the layer is independent, so the oracle's
value for those tokens is exact without evaluating the others.
"""

import numpy as np
import pytest
import torch

import oracle
import sparse_moe_ffn_route_amd as moe
import synth
from harness import dims_of, gpu_layer, logit_bound, rel_err, tolerance

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

SAMPLE_LOGITS = 32


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


def _check_grouping(inp, packed_np):
    wl = inp.wl
    d = dims_of(wl)
    T, k = wl.T, wl.top_k
    counts = torch.empty(wl.local, dtype=torch.int32, device="cuda")
    offsets = torch.empty(wl.local + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(T * k, dtype=torch.int32, device="cuda")
    inv = torch.empty(T, k, dtype=torch.int32, device="cuda")
    ws = moe.workspace(d)
    moe.moe_permute(d, torch.from_numpy(packed_np).cuda(), counts, offsets, perm, inv, ws=ws)
    ids, _ = oracle.unpack_routing(packed_np)
    c, o, p, iv = oracle.permute(ids, wl.expert_begin, wl.local)
    np.testing.assert_array_equal(counts.cpu().numpy(), c)
    np.testing.assert_array_equal(offsets.cpu().numpy(), o)
    np.testing.assert_array_equal(perm.cpu().numpy()[: int(o[-1])], p)
    np.testing.assert_array_equal(inv.cpu().numpy(), iv)
    assert int(moe.workspace_error_count(ws).cpu()[0]) == 0
    return c, o, p


def _routing(inp, g):
    """Oracle routing of every token from the GPU's fp32 logits (or the given blob), checked against the GPU's."""
    wl = inp.wl
    if wl.routing_given:
        np.testing.assert_array_equal(g["packed"], inp.packed.cpu().numpy())   # the given blob passes through
        ids, w32 = oracle.unpack_routing(g["packed"])
        return ids, w32.astype(np.float64)
    bias = None if inp.bias is None else inp.bias.cpu().numpy()
    ids, w = oracle.route(g["logits"], wl.top_k, bias=bias, renormalize=wl.renormalize)
    ids_gpu, w_gpu = oracle.unpack_routing(g["packed"])
    np.testing.assert_array_equal(ids_gpu, ids)
    np.testing.assert_allclose(w_gpu, w, rtol=0, atol=1e-6)
    # router logits on sampled tokens against the fp32 accumulation bound
    s = np.sort(np.random.default_rng(wl.T).choice(wl.T, size=min(SAMPLE_LOGITS, wl.T), replace=False))
    x_s = synth.f64(inp.x[torch.from_numpy(s).cuda()])
    wr = synth.f64(inp.w_router)
    l_ref = oracle.router_logits(x_s, wr).astype(np.float64)
    assert np.all(np.abs(g["logits"][s] - l_ref) <= logit_bound(x_s, wr, l_ref))
    return ids, w


def _oracle(inp, ids, w, tokens=None):
    """Oracle y with and without the shared expert on `tokens` (None: all), from one evaluation of the experts."""
    wl = inp.wl
    if tokens is None:
        x = synth.f64(inp.x)
    else:
        x = synth.f64(inp.x[torch.from_numpy(tokens).cuda()])
        ids, w = ids[tokens], w[tokens]
    if wl.w == "e4m3":
        res = oracle.layer_from_routing_fp8(x, ids, w, synth.ExpertViewFP8(inp), shared=synth.shared_f64(inp),
                                            expert_begin=wl.expert_begin, n_local=wl.local)
    else:
        res = oracle.layer_from_routing(x, ids, w, synth.ExpertView(inp), shared=synth.shared_f64(inp),
                                        expert_begin=wl.expert_begin, n_local=wl.local)
    routed = oracle.combine(res["out_rows"], w, res["inv_pos"])
    return res["y"], routed


def _check_layer_full(inp, tokens=None):
    """Packed weights with the shared expert (the bench's launch configuration), then row-major weights without it;
    y compared on every token (or on `tokens`)."""
    wl = inp.wl
    print(f"[full] {wl.name}: layer on the GPU", flush=True)
    g = gpu_layer(inp, packed=True)
    ids, w = _routing(inp, g)
    counts, offsets, perm = _check_grouping(inp, g["packed"])
    if callable(tokens):
        tokens = tokens(counts, offsets, perm)
    g2 = gpu_layer(inp, shared=False, packed=False)
    np.testing.assert_array_equal(g2["packed"], g["packed"])
    print(f"[full] {wl.name}: oracle on {wl.T if tokens is None else len(tokens)} tokens", flush=True)
    y_ref, routed_ref = _oracle(inp, ids, w, tokens)
    sel = slice(None) if tokens is None else tokens
    tol = tolerance(wl)
    err = rel_err(g["y"][sel], y_ref)
    assert err <= tol, f"{wl.name}: rel err {err:.3e}"
    err2 = rel_err(g2["y"][sel], routed_ref)
    assert err2 <= tol, f"{wl.name} (no shared expert): rel err {err2:.3e}"
    if wl.expert_begin != 0 or wl.local != wl.E:
        # tokens with no local expert get an all-zero partial sum
        local = ((ids >= wl.expert_begin) & (ids < wl.expert_begin + wl.local)).any(axis=1)
        none_local = np.nonzero(~local)[0]
        assert none_local.size > 0 and np.all(g["y"][none_local] == 0)
    print(f"[full] {wl.name}: rel err {err:.2e} (shared on), {err2:.2e} (routed only)", flush=True)
    return counts


def test_decode_full_size(big_layer):
    counts = _check_layer_full(_variant(big_layer, "decode_bf16"))
    assert counts.sum() == 512 * 10


def test_prefill_full_size(big_layer):
    counts = _check_layer_full(_variant(big_layer, "prefill_bf16"))
    assert counts.sum() == 8192 * 10
    assert counts.max() > 192                               # some experts fill rows 192-255 of their tile


def test_skewed_prefill_full_size(big_layer):
    counts = _check_layer_full(_variant(big_layer, "skew_prefill_bf16"))
    assert (counts == 0).sum() == 32                      # the never-chosen experts stay empty
    assert counts.max() / counts.mean() > 15              # a straggler expert many times the mean load


def _corner_tokens(counts, offsets, perm, T, n_random=24, seed=15):
    """Tokens whose grouped rows sit in the grouped GEMMs' corners: the ragged last 256-row M-tile of the three
    largest experts, rows 192-255 of every M-tile of the largest experts, and random tokens."""
    rows = []
    for e in np.argsort(-counts, kind="stable")[:3]:
        n = int(counts[e])
        last = (n - 1) // 256 * 256
        rows += list(range(offsets[e] + last, offsets[e] + n))[-8:]          # the ragged last tile's rows
        for m0 in range(0, n, 256):
            rows += [offsets[e] + r for r in range(m0 + 192, min(m0 + 256, n), 9)]
    rng = np.random.default_rng(seed)
    tok = set(perm[np.asarray(rows, dtype=np.int64)].tolist()) | set(rng.choice(T, n_random).tolist())
    return np.array(sorted(tok), dtype=np.int64)


def test_prefill32k_full_size(big_layer):
    """The 32K-token probe: experts of ~640 rows span three 256-row M-tiles."""
    wl = synth.WORKLOADS["prefill32k_bf16"]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(32768)
    x = torch.randn(wl.T, wl.D, generator=gen, device="cuda").to(torch.bfloat16)
    b = big_layer
    inp = synth.LayerInputs(wl, x, b.w_router, b.w_gate, b.w_up, b.w_down, None, None, None, b.ws_gate, b.ws_up,
                            b.ws_down, None, None)
    counts = _check_layer_full(inp, tokens=lambda c, o, p: _corner_tokens(c, o, p, wl.T))
    assert counts.sum() == 32768 * 10 and counts.min() > 256


def test_ep_share_fp8_full_size():
    wl = synth.WORKLOADS["ep_share_fp8"]
    inp = synth.make_inputs(wl, 0, "cuda")
    counts = _check_layer_full(inp)
    assert 9000 < counts.sum() < 11500                    # ~T*k*64/512 pairs are local
    del inp
    torch.cuda.empty_cache()


def test_decode_fp8_full_size():
    """The decode batch with e4m3 routed experts (router and shared expert bf16)."""
    wl = synth.WORKLOADS["decode_fp8"]
    inp = synth.make_inputs(wl, 0, "cuda")
    counts = _check_layer_full(inp)
    assert counts.sum() == 512 * 10
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
    s = np.sort(np.random.default_rng(16).choice(wl.T, size=64, replace=False))
    x_s = synth.f64(inp.x[torch.from_numpy(s).cuda()])
    ref = oracle.layer_from_routing(x_s, ids[s], w[s], synth.ExpertView(inp))
    err = rel_err(g["y"][s], ref["y"])
    assert err <= tolerance(wl), f"past-2GiB batch: sampled rel err {err:.3e}"
    del inp
    torch.cuda.empty_cache()
