"""GPU parity: every C-ABI entry point against the CPU oracle on the same seeded inputs.

Bars: routing ids, counts, offsets, permutation: bit-exact; routing weights within
1e-6 of the oracle's fp64 weights (same fp32 logits); gathered rows and E4M3 codes
bit-exact; layer output max|y - y_ref| <= tol * max|y_ref| with tol 1e-4 (fp32),
1e-2 (bf16), 3e-2 (fp8).  Sizes span several tiles with ragged tails; the
full-size workloads are checked on sampled tokens in test_gpu_full.py.
"""

import numpy as np
import pytest
import torch

import oracle
import sparse_moe_ffn_route_amd as moe
import synth
import harness
from harness import dims_of, gpu_layer, logit_bound, oracle_layer, oracle_routing, rel_err, to_np, tolerance

pytestmark = pytest.mark.gpu

W = synth.Workload

# Layer configurations: (workload, seed)
MID = {
    # fp32 tiny layer of the pages' shape family
    "tiny_fp32": synth.WORKLOADS["tiny_fp32"],
    "mid_fp32": W("mid_fp32", T=100, D=128, E=12, top_k=3, I=64, I_shared=64, act="f32", w="f32", out="f32"),
    # few rows per expert (16-row tiles), partial K block, 3 gate/up and 2 down N-tiles
    "decode_like_bf16": W("decode_like_bf16", T=96, D=256, E=64, top_k=6, I=192, I_shared=128,
                          act="bf16", w="bf16", out="bf16"),
    # ~30 rows per expert (32-row tiles, ragged second tile), 2 K blocks
    "mid_bf16": W("mid_bf16", T=300, D=512, E=40, top_k=4, I=192, I_shared=128, act="bf16", w="bf16", out="bf16"),
    # fp32 output from bf16 operands
    "mid_bf16_f32out": W("mid_bf16_f32out", T=128, D=256, E=16, top_k=2, I=128, I_shared=64,
                         act="bf16", w="bf16", out="f32"),
    # skewed popularity: a hot expert spanning many M-tiles and never-chosen experts
    "skew_bf16": W("skew_bf16", T=512, D=256, E=32, top_k=4, I=128, I_shared=64, act="bf16", w="bf16", out="bf16",
                   skew_alpha=0.8, skew_s=1.1, skew_empty=4),
    # expert-parallel slice with the router on
    "slice_bf16": W("slice_bf16", T=200, D=256, E=32, top_k=4, I=128, I_shared=0, act="bf16", w="bf16",
                    out="bf16", expert_begin=16, n_local=8),
    # fp8 slice with given routing
    "slice_fp8": W("slice_fp8", T=256, D=512, E=32, top_k=4, I=128, I_shared=0, act="bf16", w="e4m3", out="bf16",
                   expert_begin=8, n_local=8, routing_given=True),
    "slice_fp8_f32out": W("slice_fp8_f32out", T=64, D=256, E=16, top_k=3, I=64, I_shared=0, act="bf16", w="e4m3",
                          out="f32", expert_begin=0, n_local=16, routing_given=True),
    # fp8 routed experts with the router on and a bf16 shared expert (streaming and tile shapes)
    "fp8_shared": W("fp8_shared", T=200, D=512, E=32, top_k=4, I=128, I_shared=128, act="bf16", w="e4m3",
                    out="bf16"),
    "fp8_shared_tile": W("fp8_shared_tile", T=512, D=256, E=16, top_k=4, I=192, I_shared=64, act="bf16",
                         w="e4m3", out="bf16"),
    # no renormalisation; k = 1
    "norenorm_k1": W("norenorm_k1", T=77, D=128, E=8, top_k=1, I=64, I_shared=64, act="bf16", w="bf16",
                     out="bf16", renormalize=False),
    # k = E
    "k_eq_E": W("k_eq_E", T=33, D=128, E=8, top_k=8, I=64, I_shared=0, act="bf16", w="bf16", out="bf16"),
    # a single token
    "one_token": W("one_token", T=1, D=256, E=16, top_k=4, I=128, I_shared=64, act="bf16", w="bf16", out="bf16"),
    # the largest supported k: the combine sums four full batches of 8 slots
    "k_max": W("k_max", T=40, D=128, E=48, top_k=32, I=64, I_shared=64, act="bf16", w="bf16", out="bf16"),
    # k = 12 over a quarter of the experts: a ragged second batch of slots, most slots non-local
    "slice_k12_f32out": W("slice_k12_f32out", T=90, D=320, E=64, top_k=12, I=64, I_shared=0, act="bf16",
                          w="bf16", out="f32", expert_begin=40, n_local=16),
    # ~150 rows per expert (256-row tiles, one ragged M-tile each) with fp32 output from bf16 operands
    "tile_bf16_f32out": W("tile_bf16_f32out", T=600, D=256, E=16, top_k=4, I=128, I_shared=64, act="bf16",
                          w="bf16", out="f32"),
    # ~256 rows per expert at D = 1024, I = 512: the 256-row tile kernels' K loops run 16 (gate/up) and 8
    # (down) blocks, so their weight rings turn several times with a remainder; experts of 193-256 rows
    # take the 14- and 16-fragment loops, experts past 256 rows a ragged second M-tile; the 2048-token
    # router projection takes the 256-row tile shape with K splits
    "tile_wide_bf16": W("tile_wide_bf16", T=2048, D=1024, E=32, top_k=4, I=512, I_shared=256, act="bf16",
                        w="bf16", out="bf16"),
    "tile_wide_fp8": W("tile_wide_fp8", T=2048, D=1024, E=32, top_k=4, I=512, I_shared=256, act="bf16",
                       w="e4m3", out="bf16"),
    # the same width with skewed popularity: a hot expert over several M-tiles, empty experts
    "tile_wide_skew_bf16": W("tile_wide_skew_bf16", T=1536, D=1024, E=24, top_k=3, I=512, I_shared=0,
                             act="bf16", w="bf16", out="bf16", skew_alpha=0.8, skew_s=1.1, skew_empty=3),
    # fp8 expert-parallel slice at the same width with given routing (64-expert-share analogue)
    "tile_wide_fp8_slice": W("tile_wide_fp8_slice", T=4096, D=1024, E=64, top_k=8, I=512, I_shared=0,
                             act="bf16", w="e4m3", out="bf16", expert_begin=16, n_local=16, routing_given=True),
    # ragged widths past one 512-column piece: D = 704 = 512 + 192, I = 320, I_s = 192.  Every expert GEMM ends
    # on a partial N-tile (the 16-row streaming down projection's 256-channel tiles, the 256-row tiles'
    # 128-channel ones, the fused combine's last tile); the streaming K loops end on a partial block (1408 and
    # 640 bytes per row), the e4m3 tile gate/up on a lone 64-byte slice (704 bytes); a combine wave's second
    # piece is partly past D
    "ragged_decode_bf16": W("ragged_decode_bf16", T=128, D=704, E=32, top_k=4, I=320, I_shared=192, act="bf16",
                            w="bf16", out="bf16"),
    "ragged_tile_bf16": W("ragged_tile_bf16", T=2048, D=704, E=16, top_k=2, I=320, I_shared=192, act="bf16",
                          w="bf16", out="bf16"),
    "ragged_tile_fp8": W("ragged_tile_fp8", T=2048, D=704, E=16, top_k=2, I=320, I_shared=192, act="bf16",
                         w="e4m3", out="bf16"),
    "ragged_slice_fp8": W("ragged_slice_fp8", T=1024, D=704, E=16, top_k=4, I=320, I_shared=0, act="bf16",
                          w="e4m3", out="bf16", expert_begin=4, n_local=8, routing_given=True),
}


def _check_layer(wl, seed=0, shared=True, packed=False):
    inp = synth.make_inputs(wl, seed, "cpu")
    g = gpu_layer(inp, shared=shared, packed=packed)
    if not wl.routing_given:
        x64, wr64 = synth.f64(inp.x), synth.f64(inp.w_router)
        l_ref = oracle.router_logits(x64, wr64).astype(np.float64)
        bound = logit_bound(x64, wr64, l_ref)
        assert np.all(np.abs(g["logits"] - l_ref) <= bound), "router logits outside the fp32 accumulation bound"
    ref = oracle_layer(inp, g["logits"], shared=shared)
    ids_gpu, w_gpu = oracle.unpack_routing(g["packed"])
    np.testing.assert_array_equal(ids_gpu, ref["ids"])
    np.testing.assert_allclose(w_gpu, ref["weights"], rtol=0, atol=1e-6)
    err = rel_err(g["y"], ref["y"])
    tol = tolerance(wl)
    assert err <= tol, f"{wl.name}: rel err {err:.3e} > {tol}"
    return err


@pytest.mark.parametrize("name", list(MID))
def test_layer_forward_parity(name):
    _check_layer(MID[name])


@pytest.mark.parametrize("name", ["tiny_fp32", "mid_fp32", "decode_like_bf16", "mid_bf16", "mid_bf16_f32out",
                                  "skew_bf16", "slice_fp8", "slice_fp8_f32out", "fp8_shared", "fp8_shared_tile",
                                  "one_token", "tile_bf16_f32out", "tile_wide_bf16", "tile_wide_fp8",
                                  "tile_wide_skew_bf16", "tile_wide_fp8_slice", "ragged_decode_bf16",
                                  "ragged_tile_bf16", "ragged_tile_fp8", "ragged_slice_fp8"])
def test_layer_forward_parity_packed_weights(name):
    """Expert weights repacked by moe_pack_weights (fragment-major layout) give the same layer."""
    _check_layer(MID[name], seed=2, packed=True)


class _DequantView:
    """experts[e] -> dequantised (w_gate, w_up, w_down) in float64: E4M3 codes times their channel scales."""

    def __init__(self, inp):
        self.q = synth.ExpertViewFP8(inp)

    def __len__(self):
        return len(self.q)

    def __getitem__(self, e):
        (gq, gs), (uq, us), (dq, ds) = self.q[e]
        return gq * gs[:, None], uq * us[:, None], dq * ds[:, None]


@pytest.mark.parametrize("name,packed", [("mid_bf16", False), ("mid_bf16", True), ("tiny_fp32", False),
                                         ("fp8_shared", False), ("fp8_shared", True), ("slice_fp8", True)])
def test_audit_shadow_is_the_exact_layer(name, packed):
    """moe_audit's reference rows are the exact layer (stored weights, unquantised x and h) on the
    sampled tokens with the routing the layer used; its result is max |y - ref| and max |ref|."""
    wl = MID[name]
    inp = synth.make_inputs(wl, 4, "cpu")
    g = gpu_layer(inp, packed=packed)
    dev = g["dev"]
    use_shared = wl.I_shared > 0
    pw = harness.packed_weights(dev) if packed else {n: getattr(dev, n) for n in
                                                      ("w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down")}
    w = moe.make_weights(dev.w_router, pw["w_gate"], pw["w_up"], pw["w_down"], dev.s_gate, dev.s_up, dev.s_down,
                         pw["ws_gate"] if use_shared else None, pw["ws_up"] if use_shared else None,
                         pw["ws_down"] if use_shared else None)
    d = dims_of(wl, True, packed)
    rows = np.array(sorted({0, 1, wl.T // 2, wl.T - 1}), dtype=np.int32)
    sample = torch.from_numpy(rows).cuda()
    out_dt = torch.float32 if wl.out == "f32" else torch.bfloat16
    y_dev = torch.from_numpy(g["y"]).to(out_dt).cuda()          # exact: the values came from this dtype
    ref_out = torch.empty(len(rows), wl.D, dtype=torch.float32, device="cuda")
    res = moe.moe_audit(d, w, dev.x, torch.from_numpy(g["packed"]).cuda(), y_dev, sample, ref_out).cpu().numpy()
    ref = ref_out.cpu().numpy().astype(np.float64)
    ids, wts = oracle.unpack_routing(g["packed"])
    experts = _DequantView(inp) if wl.w == "e4m3" else synth.ExpertView(inp)
    exact = oracle.layer_from_routing(synth.f64(inp.x)[rows], ids[rows], wts[rows].astype(np.float64), experts,
                                      shared=synth.shared_f64(inp) if use_shared else None,
                                      expert_begin=wl.expert_begin, n_local=wl.local)["y"]
    assert rel_err(ref, exact) <= 1e-4                          # an fp32 evaluation of the exact layer
    np.testing.assert_allclose(res[1], np.abs(ref).max(), rtol=1e-6)
    np.testing.assert_allclose(res[0], np.abs(g["y"][rows] - ref).max(), rtol=1e-5, atol=1e-7)
    bound = 0.1 if wl.w == "e4m3" else tolerance(wl)            # fp8 quantisation shows, a few percent
    assert res[0] / res[1] <= bound


def test_hbm_read_probe_reads_every_byte_once():
    """The XOR of the probe's checksum words is the XOR of every 32-bit word of the buffer."""
    rng = np.random.default_rng(4)
    words = rng.integers(-2 ** 31, 2 ** 31, size=(1 << 18) + 12, dtype=np.int64).astype(np.int32)
    buf = torch.from_numpy(words).cuda()
    sink = torch.zeros(moe.HBM_PROBE_SINK_WORDS, dtype=torch.int32, device="cuda")
    moe.moe_hbm_read_probe(buf, sink)
    got = np.bitwise_xor.reduce(sink.cpu().numpy())
    assert got == np.bitwise_xor.reduce(words)


@pytest.mark.parametrize("dtype", ["bf16", "e4m3"])
def test_mfma_peak_probe_runs(dtype):
    """The MFMA probe completes and leaves finite, non-zero sums (its work was not dropped)."""
    sink, flop = moe.moe_mfma_peak_probe(dtype, 64)
    torch.cuda.synchronize()
    s = sink.cpu().numpy()
    assert flop == moe.MFMA_PROBE_BLOCKS * 4 * 8 * 64 * (16384 if dtype == "bf16" else 65536)
    assert np.isfinite(s).all() and (s != 0).all()


def test_pack_weights_layout():
    """moe_pack_weights places row (16 f + l % 16), bytes [64 s + 16 (l / 16), +16) at run (f, s), chunk l."""
    rng = np.random.default_rng(3)
    n, rows, cols = 3, 48, 256
    src = torch.from_numpy(rng.integers(0, 2 ** 16, (n, rows, cols), dtype=np.int64).astype(np.int16))
    src = src.view(torch.bfloat16).cuda()
    dst = moe.moe_pack_weights(src).cpu().view(torch.int16).numpy()
    a = src.cpu().view(torch.int16).numpy().reshape(n, rows // 16, 16, cols * 2 // 64, 4, 8)  # [n][f][r][s][g][8 elems]
    expect = a.transpose(0, 1, 3, 4, 2, 5).reshape(-1)                                        # [n][f][s][g][r][8]
    np.testing.assert_array_equal(dst.reshape(-1), expect)


@pytest.mark.parametrize("name", ["mid_bf16", "decode_like_bf16", "tiny_fp32", "skew_bf16", "tile_wide_bf16",
                                  "tile_wide_fp8", "fp8_shared_tile", "ragged_decode_bf16", "ragged_tile_bf16",
                                  "ragged_tile_fp8"])
def test_layer_forward_parity_without_shared_expert(name):
    """The shared expert dominates y; without it a routed-path error cannot hide under the tolerance."""
    _check_layer(MID[name], seed=1, shared=False)


def test_layer_forward_two_calls_reuse_workspace():
    wl = MID["mid_bf16"]
    inp = synth.make_inputs(wl, 3, "cpu")
    ws = moe.workspace(dims_of(wl))
    a = gpu_layer(inp, ws=ws)
    b = gpu_layer(inp, ws=ws)
    np.testing.assert_array_equal(a["y"], b["y"])           # deterministic
    np.testing.assert_array_equal(a["packed"], b["packed"])


@pytest.mark.parametrize("name", ["decode_like_bf16", "fp8_shared_tile"])
def test_layer_forward_runs_on_the_given_stream(name):
    """Every launch of the layer goes to the stream it is given: on a second stream (default priority, ordered
    after the inputs by an explicit wait), passed by the current-stream context and as an argument, y and the
    routing blob equal the default-stream call's bit for bit."""
    wl = MID[name]
    ref = gpu_layer(synth.make_inputs(wl, 5, "cpu"))
    dev = ref["dev"]
    d = dims_of(wl)
    w = moe.make_weights(dev.w_router, dev.w_gate, dev.w_up, dev.w_down, dev.s_gate, dev.s_up, dev.s_down,
                         dev.ws_gate, dev.ws_up, dev.ws_down)
    side = torch.cuda.Stream()
    outs = []
    for by_context in (True, False):
        ws = moe.workspace(d)
        y = torch.full((wl.T, wl.D), float("nan"), dtype=harness._OUT_TORCH[wl.out], device="cuda")
        logits = None if wl.routing_given else torch.empty(wl.T, wl.E, dtype=torch.float32, device="cuda")
        blob = torch.full((wl.T, 2, wl.top_k), -7, dtype=torch.int32, device="cuda")
        side.wait_stream(torch.cuda.current_stream())
        if by_context:
            with torch.cuda.stream(side):
                moe.moe_layer_forward(d, w, dev.x, dev.packed, dev.bias, y, logits, blob, ws)
        else:
            moe.moe_layer_forward(d, w, dev.x, dev.packed, dev.bias, y, logits, blob, ws, stream=side)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        outs.append((harness.to_np(y), blob.cpu().numpy()))
    for y, blob in outs:
        np.testing.assert_array_equal(y, ref["y"])
        np.testing.assert_array_equal(blob, ref["packed"])


def test_stage_events_time_the_same_layer():
    """Stage events only mark the stream: y is bit-identical, and the marks are in stage order."""
    wl = MID["decode_like_bf16"]
    dev = synth.make_inputs(wl, 3, "cpu").to("cuda")
    d = dims_of(wl)
    ws = moe.workspace(d)
    w = moe.make_weights(dev.w_router, dev.w_gate, dev.w_up, dev.w_down, None, None, None,
                         dev.ws_gate, dev.ws_up, dev.ws_down)
    ys = []
    for timed in (False, True):
        y = torch.empty(wl.T, wl.D, dtype=torch.bfloat16, device="cuda")
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(moe.STAGE_EVENTS)] if timed else None
        moe.moe_layer_forward(d, w, dev.x, None, None, y, stage_events=evs, ws=ws)
        torch.cuda.synchronize()
        ys.append(y.cpu())
    assert len(moe.STAGES) == moe.STAGE_EVENTS - 1
    spans = [evs[i].elapsed_time(evs[i + 1]) for i in range(moe.STAGE_EVENTS - 1)]
    assert all(t >= 0.0 for t in spans), spans
    assert spans[moe.STAGES.index("shared")] > 0.0       # the shared expert has launches of its own
    torch.testing.assert_close(ys[0], ys[1], rtol=0, atol=0)


def test_expert_parallel_slices_sum_to_full_layer():
    """Eight slices run one after another sum to the full routed layer (what a reduce-scatter adds)."""
    full = W("ep_full", T=256, D=256, E=64, top_k=4, I=128, I_shared=0, act="bf16", w="bf16", out="f32",
             routing_given=True)
    inp = synth.make_inputs(full, 5, "cpu")
    y_full = gpu_layer(inp)["y"]
    total = np.zeros_like(y_full)
    for b in range(0, 64, 8):
        wl = full.replace(expert_begin=b, n_local=8)
        part = synth.LayerInputs(wl, inp.x, None, inp.w_gate[b:b + 8].contiguous(), inp.w_up[b:b + 8].contiguous(),
                                 inp.w_down[b:b + 8].contiguous(), packed=inp.packed)
        total += gpu_layer(part)["y"]
    assert rel_err(total, y_full) < 1e-5


# ---------------------------------------------------------------------------
# moe_route
# ---------------------------------------------------------------------------

ROUTE_CASES = [
    # (T, E, k, kind, renormalize)
    (1000, 512, 10, "normal", True),
    (700, 512, 10, "ties", True),
    (300, 100, 7, "normal", True),
    (257, 1024, 32, "normal", True),
    (64, 16, 2, "ties", False),
    (129, 32, 32, "normal", True),
    (50, 512, 10, "bias_inf", True),
    (31, 8, 1, "ties", True),
]


@pytest.mark.parametrize("T,E,k,kind,renorm", ROUTE_CASES)
def test_route_from_given_logits(T, E, k, kind, renorm):
    rng = np.random.default_rng(T * 7 + E)
    if kind == "ties":
        logits = rng.choice(np.array([-1.0, -0.0, 0.0, 0.5, 0.5, 3.0], np.float32), size=(T, E))
    else:
        logits = rng.standard_normal((T, E)).astype(np.float32)
    bias = None
    if kind == "bias_inf":
        bias = (rng.standard_normal(E) * 0.5).astype(np.float32)
        bias[rng.choice(E, E // 4, replace=False)] = -np.inf
    d = moe.make_dims(T, 64, E, k, 64, renormalize=renorm)
    lg = torch.from_numpy(logits).cuda()
    packed = torch.empty(T, 2, k, dtype=torch.int32, device="cuda")
    moe.moe_route(d, None, None, lg, None if bias is None else torch.from_numpy(bias).cuda(), packed)
    ids_gpu, w_gpu = oracle.unpack_routing(packed.cpu().numpy())
    ids, w = oracle.route(logits, k, bias=bias, renormalize=renorm)
    np.testing.assert_array_equal(ids_gpu, ids)
    np.testing.assert_allclose(w_gpu, w, rtol=0, atol=1e-6)


@pytest.mark.parametrize("split", [False, True])
@pytest.mark.parametrize("T,D,E,k", [(333, 512, 128, 6), (3000, 512, 200, 8)])
def test_route_with_router_projection_bf16(split, T, D, E, k):
    """Without scratch the projection is one pass over D; with it, D is split into
    partial products summed in a fixed order by the routing kernel.  333 tokens take the
    32-row streaming tiles, 3000 the 256-row tiles (ragged last tile, E below one N-tile)."""
    rng = np.random.default_rng(1)
    x = torch.from_numpy(rng.standard_normal((T, D)).astype(np.float32)).to(torch.bfloat16)
    wr = torch.from_numpy((rng.standard_normal((E, D)) / np.sqrt(D)).astype(np.float32)).to(torch.bfloat16)
    d = moe.make_dims(T, D, E, k, 64)
    logits = torch.empty(T, E, dtype=torch.float32, device="cuda")
    packed = torch.empty(T, 2, k, dtype=torch.int32, device="cuda")
    moe.moe_route(d, x.cuda(), wr.cuda(), logits, None, packed, ws=moe.workspace(d) if split else None)
    x64, w64 = to_np(x), to_np(wr)
    l_ref = oracle.router_logits(x64, w64).astype(np.float64)
    lg = logits.cpu().numpy()
    assert np.all(np.abs(lg - l_ref) <= logit_bound(x64, w64, l_ref))
    ids, w = oracle.route(lg, k)
    ids_gpu, w_gpu = oracle.unpack_routing(packed.cpu().numpy())
    np.testing.assert_array_equal(ids_gpu, ids)
    np.testing.assert_allclose(w_gpu, w, rtol=0, atol=1e-6)


@pytest.mark.parametrize("T,D,E,k,act,renorm,biased", [
    (333, 512, 128, 6, "bf16", True, False),     # ragged last 16-token block, two 64-expert slices
    (3000, 512, 200, 8, "bf16", True, True),     # 64-token blocks, 128-expert slices, bias, E not a multiple of 64
    (100, 256, 64, 4, "f32", False, False),      # fp32 operands, no renormalisation (slice softmax sums)
    (2500, 256, 300, 12, "bf16", False, True),   # no renormalisation with bias over three 128-expert slices
    (512, 4096, 512, 10, "bf16", True, False),   # the decode router shape
    (77, 128, 1024, 32, "bf16", True, False),    # the largest E and k: 16 slices x 32 candidates per token
    (40, 128, 80, 32, "bf16", True, True),       # a slice with fewer experts than k (sentinel candidates)
])
def test_route_fused_matches_definition(T, D, E, k, act, renorm, biased):
    """The fused router: logits within the fp32 bound, routing bit-exact from its own logits,
    and the same blob whether or not the logits are copied out."""
    rng = np.random.default_rng(T + E)
    dt = torch.float32 if act == "f32" else torch.bfloat16
    x = torch.from_numpy(rng.standard_normal((T, D)).astype(np.float32)).to(dt)
    wr = torch.from_numpy((rng.standard_normal((E, D)) / np.sqrt(D)).astype(np.float32)).to(dt)
    bias = torch.from_numpy(rng.standard_normal(E).astype(np.float32) * 0.5) if biased else None
    d = moe.make_dims(T, D, E, k, 64, act=act, w=act, out=act, renormalize=renorm)
    logits = torch.empty(T, E, dtype=torch.float32, device="cuda")
    packed = torch.empty(T, 2, k, dtype=torch.int32, device="cuda")
    moe.moe_route_fused(d, x.cuda(), wr.cuda(), logits, None if bias is None else bias.cuda(), packed)
    x64, w64 = to_np(x), to_np(wr)
    l_ref = oracle.router_logits(x64, w64).astype(np.float64)
    lg = logits.cpu().numpy()
    assert np.all(np.abs(lg - l_ref) <= logit_bound(x64, w64, l_ref))
    ids, w = oracle.route(lg, k, bias=None if bias is None else bias.numpy(), renormalize=renorm)
    ids_gpu, w_gpu = oracle.unpack_routing(packed.cpu().numpy())
    np.testing.assert_array_equal(ids_gpu, ids)
    np.testing.assert_allclose(w_gpu, w, rtol=0, atol=1e-6)
    packed2 = torch.empty_like(packed)
    moe.moe_route_fused(d, x.cuda(), wr.cuda(), None, None if bias is None else bias.cuda(), packed2)
    np.testing.assert_array_equal(packed2.cpu().numpy(), packed.cpu().numpy())


# ---------------------------------------------------------------------------
# moe_permute
# ---------------------------------------------------------------------------

PERM_CASES = [
    # (T, k, E, begin, n_local, junk): junk adds out-of-range ids and repeats
    (512, 10, 512, 0, 512, False),
    (5000, 10, 512, 64, 64, False),
    (3001, 4, 100, 0, 100, True),
    (1, 1, 4, 0, 4, False),
    (2049, 8, 1024, 0, 1024, False),
    (777, 3, 16, 5, 1, True),
    (12000, 10, 512, 128, 64, True),   # beyond the one-workgroup path: histogram / scan / scatter kernels
]


def _packed_blob(rng, T, k, E, junk):
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int32)
    if junk:
        m = rng.random((T, k)) < 0.1
        ids[m] = rng.integers(-3, E + 3, m.sum())
    w = rng.random((T, k)).astype(np.float32)
    return oracle.pack_routing(ids, w), ids


@pytest.mark.parametrize("T,k,E,begin,n_local,junk", PERM_CASES)
def test_permute_bit_exact(T, k, E, begin, n_local, junk):
    rng = np.random.default_rng(T + k)
    packed, ids = _packed_blob(rng, T, k, E, junk)
    d = moe.make_dims(T, 64, E, k, 64, expert_begin=begin, n_local=n_local)
    counts = torch.empty(n_local, dtype=torch.int32, device="cuda")
    offsets = torch.empty(n_local + 1, dtype=torch.int32, device="cuda")
    perm = torch.full((T * k,), -7, dtype=torch.int32, device="cuda")
    inv = torch.empty(T, k, dtype=torch.int32, device="cuda")
    ws = moe.workspace(d)
    moe.moe_permute(d, torch.from_numpy(packed).cuda(), counts, offsets, perm, inv, ws=ws)
    c, o, p, iv = oracle.permute(ids, begin, n_local)
    np.testing.assert_array_equal(counts.cpu().numpy(), c)
    np.testing.assert_array_equal(offsets.cpu().numpy(), o)
    n_a = int(o[-1])
    np.testing.assert_array_equal(perm.cpu().numpy()[:n_a], p)
    np.testing.assert_array_equal(inv.cpu().numpy(), iv)
    # the workspace error word counts the ids outside [0, E), and is rewritten by the next call
    n_bad = int(((ids < 0) | (ids >= E)).sum())
    assert (n_bad > 0) == junk
    assert int(moe.workspace_error_count(ws).cpu()[0]) == n_bad
    clean = np.where((ids < 0) | (ids >= E), 0, ids).astype(np.int32)
    moe.moe_permute(d, torch.from_numpy(oracle.pack_routing(clean, np.ones(ids.shape, np.float32))).cuda(), counts,
                    offsets, perm, inv, ws=ws)
    assert int(moe.workspace_error_count(ws).cpu()[0]) == 0


def test_layer_with_corrupt_given_blob_skips_and_counts_bad_ids():
    """A given blob with ids outside [0, E): those pairs contribute nothing and are counted."""
    wl = MID["slice_fp8"]
    inp = synth.make_inputs(wl, 7, "cpu")
    ids, w32 = oracle.unpack_routing(inp.packed.numpy())
    rng = np.random.default_rng(8)
    m = rng.random(ids.shape) < 0.15
    ids = ids.copy()
    ids[m] = np.where(rng.random(int(m.sum())) < 0.5, -1 - rng.integers(0, 5, int(m.sum())),
                      wl.E + rng.integers(0, 5, int(m.sum())))
    inp.packed = torch.from_numpy(oracle.pack_routing(ids, w32))
    d = dims_of(wl)
    ws = moe.workspace(d)
    g = gpu_layer(inp, ws=ws)
    assert int(moe.workspace_error_count(ws).cpu()[0]) == int(m.sum())
    ref = oracle_layer(inp)
    assert rel_err(g["y"], ref["y"]) <= tolerance(wl)


@pytest.mark.parametrize("T,k,E,begin,n_local", [(300, 4, 24, 0, 24), (2600, 4, 32, 8, 16)])
def test_permute_gathers_rows_and_quantises_fp8(T, k, E, begin, n_local):
    """Gathered rows through moe_permute.  The second case has 10,400 pairs (the multi-workgroup grouping, whose
    ranking launch also quantises x) and a slice, so some tokens have no local slot."""
    D = 256
    rng = np.random.default_rng(2)
    packed, ids = _packed_blob(rng, T, k, E, False)
    x = torch.from_numpy(rng.standard_normal((T, D)).astype(np.float32)).to(torch.bfloat16)
    x[7] = 0                                                 # an all-zero token: scale 1
    c, o, p, iv = oracle.permute(ids, begin, n_local)
    n_a = int(o[-1])
    # bf16 gather: every local slot's row is its token's row
    d = moe.make_dims(T, D, E, k, 64, expert_begin=begin, n_local=n_local)
    counts = torch.empty(n_local, dtype=torch.int32, device="cuda")
    offsets = torch.empty(n_local + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(T * k, dtype=torch.int32, device="cuda")
    inv = torch.empty(T, k, dtype=torch.int32, device="cuda")
    xp = torch.empty(T * k, D, dtype=torch.bfloat16, device="cuda")
    moe.moe_permute(d, torch.from_numpy(packed).cuda(), counts, offsets, perm, inv, x.cuda(), xp, None,
                    ws=moe.workspace(d))
    np.testing.assert_array_equal(inv.cpu().numpy(), iv)
    np.testing.assert_array_equal(xp.cpu()[:n_a].view(torch.int16).numpy(),
                                  x[torch.from_numpy(p.astype(np.int64))].view(torch.int16).numpy())
    # fp8 gather: per-token E4M3 codes and scales, bit-exact against the oracle's quantiser
    d8 = moe.make_dims(T, D, E, k, 64, expert_begin=begin, n_local=n_local, w="e4m3")
    xq = torch.empty(T * k, D, dtype=torch.uint8, device="cuda")
    xs = torch.empty(T * k, dtype=torch.float32, device="cuda")
    moe.moe_permute(d8, torch.from_numpy(packed).cuda(), counts, offsets, perm, inv, x.cuda(), xq, xs,
                    ws=moe.workspace(d8))
    q_ref, s_ref = oracle.quantize_rows_e4m3(to_np(x))
    codes_ref = oracle.e4m3_encode(q_ref)
    np.testing.assert_array_equal(xq.cpu().numpy()[:n_a], codes_ref[p])
    np.testing.assert_array_equal(xs.cpu().numpy()[:n_a], s_ref[p])


# ---------------------------------------------------------------------------
# moe_grouped_ffn and moe_unpermute_combine
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["mid_bf16", "decode_like_bf16", "mid_fp32"])
def test_grouped_ffn_gather_and_grouped_rows_agree_with_oracle(name):
    wl = MID[name]
    inp = synth.make_inputs(wl, 4, "cpu")
    dev = inp.to("cuda")
    rng = np.random.default_rng(4)
    packed, ids = _packed_blob(rng, wl.T, wl.top_k, wl.E, False)
    d = dims_of(wl, shared=False)
    ws = moe.workspace(d)
    T, k, D = wl.T, wl.top_k, wl.D
    counts = torch.empty(wl.local, dtype=torch.int32, device="cuda")
    offsets = torch.empty(wl.local + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(T * k, dtype=torch.int32, device="cuda")
    inv = torch.empty(T, k, dtype=torch.int32, device="cuda")
    xp = torch.empty(T * k, D, dtype=dev.x.dtype, device="cuda")
    moe.moe_permute(d, torch.from_numpy(packed).cuda(), counts, offsets, perm, inv, dev.x, xp, None, ws=ws)
    out_dt = torch.float32 if wl.out == "f32" else torch.bfloat16
    out_a = torch.empty(T * k, D, dtype=out_dt, device="cuda")
    out_b = torch.empty(T * k, D, dtype=out_dt, device="cuda")
    moe.moe_grouped_ffn(d, dev.x, None, perm, offsets, dev.w_gate, dev.w_up, dev.w_down, None, None, None, out_a, ws)
    moe.moe_grouped_ffn(d, xp, None, None, offsets, dev.w_gate, dev.w_up, dev.w_down, None, None, None, out_b, ws)
    torch.cuda.synchronize()
    n_a = int(offsets[-1].item())
    a, b = to_np(out_a[:n_a]), to_np(out_b[:n_a])
    np.testing.assert_array_equal(a, b)                      # same sums in the same order
    c, o, p, iv = oracle.permute(ids, 0, wl.local)
    x64 = synth.f64(inp.x)
    ev = synth.ExpertView(inp)
    ref = np.zeros((n_a, D))
    for e in range(wl.local):
        if o[e] < o[e + 1]:
            ref[o[e]:o[e + 1]] = oracle.swiglu_expert(x64[p[o[e]:o[e + 1]]], *ev[e])
    assert rel_err(a, ref) <= tolerance(wl)
    # combine the grouped outputs
    y = torch.empty(T, D, dtype=out_dt, device="cuda")
    moe.moe_unpermute_combine(d, out_a, torch.from_numpy(packed).cuda(), inv, None, y)
    _, w32 = oracle.unpack_routing(packed)
    y_ref = oracle.combine(a, w32.astype(np.float64), iv)    # same (rounded) rows: only the sum is checked
    np.testing.assert_allclose(to_np(y), y_ref, rtol=0, atol=(1e-6 if wl.out == "f32" else 2 ** -8) * np.abs(y_ref).max())


def test_shared_expert_alone_through_grouped_ffn():
    wl = MID["mid_bf16"]
    inp = synth.make_inputs(wl, 6, "cpu")
    dev = inp.to("cuda")
    d = moe.make_dims(wl.T, wl.D, 1, 1, wl.I_shared, act="bf16", w="bf16", out="bf16")
    offsets = torch.tensor([0, wl.T], dtype=torch.int32, device="cuda")
    out = torch.empty(wl.T, wl.D, dtype=torch.bfloat16, device="cuda")
    moe.moe_grouped_ffn(d, dev.x, None, None, offsets, dev.ws_gate, dev.ws_up, dev.ws_down, None, None, None, out,
                        moe.workspace(d))
    ref = oracle.swiglu_expert(synth.f64(inp.x), *synth.shared_f64(inp))
    assert rel_err(to_np(out), ref) <= 1e-2
