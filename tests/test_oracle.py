"""Pins for the CPU oracle (no GPU).

Each test ties the oracle to something other than itself: a library
routine (torch casts, torch's silu / linear, scipy's softmax), a
brute-force formulation (dense evaluation of every expert masked by the
routing, pure-Python loops for selection and grouping), a closed form
(the hand-derived worked example), or an invariant of the method.
"""

import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch
from hypothesis import given, settings, strategies as st

import oracle
from oracle import numerics

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# Storage grids
# ---------------------------------------------------------------------------

def _spread_f32(n, seed):
    rng = np.random.default_rng(seed)
    mant = rng.random(n) + 0.5
    exp = rng.integers(-140, 128, n)
    sign = rng.choice([-1.0, 1.0], n)
    with np.errstate(over="ignore"):
        return (sign * np.ldexp(mant, exp)).astype(np.float32)


def test_bf16_round_matches_torch_cast():
    a = _spread_f32(200_000, 1)
    specials = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2 ** -130, 0.0, -0.0,
                         np.inf, -np.inf, 3.3895e38, 3.4e38, 1e-45], dtype=np.float32)
    a = np.concatenate([a, specials])
    ref = torch.from_numpy(a).to(torch.bfloat16).to(torch.float64).numpy()
    got = numerics.bf16_round(a)
    assert np.array_equal(np.signbit(got), np.signbit(ref))
    np.testing.assert_array_equal(got, ref)
    # ties go to even
    assert numerics.bf16_round(np.float32(1 + 2 ** -8)) == 1.0
    assert numerics.bf16_round(np.float32(1 + 3 * 2 ** -8)) == 1 + 2 ** -6


def test_e4m3_codes_decode_like_torch_and_round_trip():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = numerics.e4m3_decode(codes)
    finite = ~np.isnan(ref)
    assert np.array_equal(np.isnan(got), ~finite)
    np.testing.assert_array_equal(got[finite], ref[finite])
    # every finite code is a fixed point of rounding and encodes back to itself
    np.testing.assert_array_equal(numerics.e4m3_round(got[finite]), got[finite])
    np.testing.assert_array_equal(numerics.e4m3_encode(got[finite]), codes[finite])
    assert np.nanmax(got) == 448.0 and np.nanmin(got) == -448.0


def test_e4m3_round_matches_torch_cast_after_clamp():
    rng = np.random.default_rng(2)
    a = np.concatenate([
        rng.standard_normal(100_000) * 10.0 ** rng.integers(-4, 3, 100_000),
        rng.uniform(-600, 600, 20_000),
        # ties: between 1 and 1.125; between subnormals; at the top (464: 448 vs the NaN slot)
        [1 + 1 / 16, 1 + 3 / 16, 2 ** -10, 3 * 2 ** -10, 464.0, -464.0, 449.0, 1000.0, 0.0, -0.0],
    ]).astype(np.float32)
    ref = torch.from_numpy(np.clip(a, -448, 448)).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = numerics.e4m3_round(a.astype(np.float64))
    np.testing.assert_array_equal(got, ref)
    assert numerics.e4m3_round(1 + 1 / 16) == 1.0
    assert numerics.e4m3_round(1 + 3 / 16) == 1.25
    assert numerics.e4m3_round(2 ** -10) == 0.0
    assert numerics.e4m3_round(3 * 2 ** -10) == 2 ** -8


def test_quantize_rows_matches_torch_codes():
    rng = np.random.default_rng(3)
    x = numerics.bf16_round(rng.standard_normal((37, 96)).astype(np.float32))
    x[5] = 0.0                                           # all-zero row: scale 1
    q, s = oracle.quantize_rows_e4m3(x)
    x32 = x.astype(np.float32)
    amax = np.abs(x32).max(axis=1)
    s_ref = np.where(amax == 0, np.float32(1), amax / np.float32(448)).astype(np.float32)
    np.testing.assert_array_equal(s, s_ref)
    div = torch.from_numpy(x32) / torch.from_numpy(s_ref)[:, None]      # fp32 division in torch
    ref = div.clamp(-448, 448).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(q, ref)
    # the row maximum maps to the top of the grid
    assert np.all(np.abs(q[np.arange(37) != 5]).max(axis=1) == 448.0)


# ---------------------------------------------------------------------------
# Routing
# ---------------------------------------------------------------------------

def _select_by_loops(keys_row, k):
    """Top-k by repeated scans: larger key wins, equal key -> lower index (pure Python)."""
    taken = []
    for _ in range(k):
        best = None
        for e, v in enumerate(keys_row):
            if e in taken:
                continue
            if best is None or v > keys_row[best]:
                best = e
        taken.append(best)
    return taken


@settings(max_examples=60, deadline=None)
@given(T=st.integers(1, 6), E=st.integers(1, 20), data=st.data())
def test_route_selection_brute_force(T, E, data):
    k = data.draw(st.integers(1, E))
    seed = data.draw(st.integers(0, 2 ** 31 - 1))
    rng = np.random.default_rng(seed)
    # few distinct values so that ties are common; signed zeros included
    vals = np.array([-1.5, -0.0, 0.0, 0.25, 0.25, 2.0, -np.inf], dtype=np.float32)
    logits = rng.choice(vals, size=(T, E)).astype(np.float32)
    # guarantee k finite keys per token
    for t in range(T):
        fin = np.isfinite(logits[t])
        if fin.sum() < k:
            logits[t, np.nonzero(~fin)[0][: k - fin.sum()]] = 0.5
    ids, w = oracle.route(logits, k)
    for t in range(T):
        assert ids[t].tolist() == _select_by_loops(logits[t].tolist(), k)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-12)


def test_route_all_equal_keys():
    logits = np.full((5, 16), 0.75, dtype=np.float32)
    ids, w = oracle.route(logits, 4)
    assert (ids == np.arange(4)).all()
    assert (w == 0.25).all()


def test_route_k1_weight_is_one():
    rng = np.random.default_rng(4)
    logits = rng.standard_normal((50, 12)).astype(np.float32)
    ids, w = oracle.route(logits, 1)
    np.testing.assert_array_equal(ids[:, 0], np.argmax(logits, axis=1))
    assert (w == 1.0).all()


def test_route_k_equals_E_is_full_softmax():
    rng = np.random.default_rng(5)
    logits = (3 * rng.standard_normal((20, 9))).astype(np.float32)
    ids, w = oracle.route(logits, 9)
    ref = scipy.special.softmax(logits.astype(np.float64), axis=1)
    np.testing.assert_allclose(w, np.take_along_axis(ref, ids, axis=1), rtol=1e-13, atol=0)
    # slots are in descending key order
    assert np.all(np.diff(np.take_along_axis(logits, ids, axis=1), axis=1) <= 0)


def test_route_without_renormalisation_keeps_softmax_entries():
    rng = np.random.default_rng(6)
    logits = rng.standard_normal((20, 32)).astype(np.float32)
    ids, w = oracle.route(logits, 5, renormalize=False)
    ref = scipy.special.softmax(logits.astype(np.float64), axis=1)
    np.testing.assert_allclose(w, np.take_along_axis(ref, ids, axis=1), rtol=1e-13, atol=0)


def test_route_bias_shifts_and_excludes():
    rng = np.random.default_rng(7)
    logits = rng.standard_normal((40, 16)).astype(np.float32)
    bias = np.zeros(16, np.float32)
    bias[3] = 100.0            # always the top choice
    bias[[0, 1, 2]] = -np.inf  # never chosen
    ids, w = oracle.route(logits, 3, bias=bias)
    assert (ids[:, 0] == 3).all()
    assert not np.isin(ids, [0, 1, 2]).any()
    # renormalised weights: the biased expert holds essentially all the mass
    assert (w[:, 0] > 1 - 1e-12).all()


def test_pack_routing_plane_order_against_a_hand_written_blob():
    """Plane 0 holds the ids, plane 1 the IEEE binary32 bit patterns of the weights, token-major
    ([T][2][k]); the words below are written out by hand (0.75 = 0x3F400000, 0.25 = 0x3E800000,
    0.5 = 0x3F000000, 1.0 = 0x3F800000, -0.0 = 0x80000000)."""
    ids = np.array([[3, 1], [0, 7]], dtype=np.int32)
    w = np.array([[0.75, 0.25], [1.0, -0.0]], dtype=np.float32)
    blob = oracle.pack_routing(ids, w)
    expect = np.array([[[3, 1], [0x3F400000, 0x3E800000]],
                       [[0, 7], [0x3F800000, -0x80000000]]], dtype=np.int64).astype(np.int32)
    assert blob.dtype == np.int32 and blob.shape == (2, 2, 2)
    np.testing.assert_array_equal(blob, expect)
    i2, w2 = oracle.unpack_routing(np.array([[[5, 6], [0x3F000000, 0x3F800000]]], dtype=np.int32))
    np.testing.assert_array_equal(i2, [[5, 6]])
    np.testing.assert_array_equal(w2, np.array([[0.5, 1.0]], dtype=np.float32))


def test_pack_unpack_round_trip_bits():
    rng = np.random.default_rng(8)
    ids = rng.integers(0, 512, (33, 10)).astype(np.int32)
    w = rng.random((33, 10)).astype(np.float32)
    w[0, 0] = -0.0
    packed = oracle.pack_routing(ids, w)
    assert packed.shape == (33, 2, 10) and packed.dtype == np.int32
    i2, w2 = oracle.unpack_routing(packed)
    np.testing.assert_array_equal(i2, ids)
    np.testing.assert_array_equal(w2.view(np.int32), w.view(np.int32))


# ---------------------------------------------------------------------------
# Permutation
# ---------------------------------------------------------------------------

def _group_by_loops(ids, begin, n_local):
    T = len(ids)
    k = len(ids[0]) if T else 0
    counts, perm_token = [], []
    inv = [[-1] * k for _ in range(T)]
    for e in range(n_local):
        c = 0
        for t in range(T):
            for j in range(k):
                if ids[t][j] == begin + e:
                    inv[t][j] = len(perm_token)
                    perm_token.append(t)
                    c += 1
        counts.append(c)
    return counts, perm_token, inv


@settings(max_examples=60, deadline=None)
@given(T=st.integers(0, 9), k=st.integers(1, 4), E=st.integers(1, 12), data=st.data())
def test_permute_brute_force(T, k, E, data):
    begin = data.draw(st.integers(0, E - 1))
    n_local = data.draw(st.integers(1, E - begin))
    seed = data.draw(st.integers(0, 2 ** 31 - 1))
    rng = np.random.default_rng(seed)
    # caller-supplied blobs may repeat an expert within a token or hold ids out of range
    ids = rng.integers(-2, E + 2, (T, k))
    counts, offsets, perm_token, inv_pos = oracle.permute(ids, begin, n_local)
    c_ref, p_ref, inv_ref = _group_by_loops(ids.tolist(), begin, n_local)
    assert counts.tolist() == c_ref
    assert perm_token.tolist() == p_ref
    assert inv_pos.tolist() == inv_ref
    assert offsets[0] == 0 and offsets[-1] == len(p_ref)
    np.testing.assert_array_equal(np.diff(offsets), counts)


def test_permute_invariants_and_identity():
    rng = np.random.default_rng(9)
    T, E, k, D = 300, 64, 6, 8
    logits = rng.standard_normal((T, E)).astype(np.float32)
    ids, _ = oracle.route(logits, k)
    counts, offsets, perm_token, inv_pos = oracle.permute(ids, 0, E)
    assert counts.sum() == T * k and offsets[-1] == T * k
    for e in range(E):
        seg = perm_token[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0)              # tokens ascending inside an expert
    x = rng.standard_normal((T, D))
    x_perm = x[perm_token]                           # permute
    for t in range(T):                               # unpermute is the inverse
        for j in range(k):
            assert np.array_equal(x_perm[inv_pos[t, j]], x[t])
    # the permutation visits every (t, j) exactly once
    assert sorted(inv_pos.reshape(-1).tolist()) == list(range(T * k))


def test_permute_slices_partition_the_full_grouping():
    rng = np.random.default_rng(10)
    T, E, k = 200, 64, 4
    ids, _ = oracle.route(rng.standard_normal((T, E)).astype(np.float32), k)
    full = oracle.permute(ids, 0, E)
    seen = np.full((T, k), -1)
    base = 0
    for b in range(0, E, 16):
        c, o, p, inv = oracle.permute(ids, b, 16)
        np.testing.assert_array_equal(c, full[0][b:b + 16])
        np.testing.assert_array_equal(p, full[2][full[1][b]:full[1][b + 16]])
        m = inv >= 0
        assert (seen[m] == -1).all()
        seen[m] = inv[m] + base
        base += int(o[-1])
    np.testing.assert_array_equal(seen, full[3])


# ---------------------------------------------------------------------------
# Experts, combine, whole layer
# ---------------------------------------------------------------------------

def test_silu_matches_torch():
    z = np.concatenate([np.linspace(-800, 800, 4001), [-0.0, 0.0, 1e-300, -1e-300]])
    ref = torch.nn.functional.silu(torch.from_numpy(z)).numpy()
    np.testing.assert_allclose(oracle.silu(z), ref, rtol=1e-15, atol=1e-300)


def _rand_layer(rng, T, D, E, I, Is):
    x = rng.standard_normal((T, D))
    wr = rng.standard_normal((E, D)) / math.sqrt(D)
    wg = rng.standard_normal((E, I, D)) / math.sqrt(D)
    wu = rng.standard_normal((E, I, D)) / math.sqrt(D)
    wd = rng.standard_normal((E, D, I)) / math.sqrt(I)
    shared = None
    if Is:
        shared = (rng.standard_normal((Is, D)) / math.sqrt(D), rng.standard_normal((Is, D)) / math.sqrt(D),
                  rng.standard_normal((D, Is)) / math.sqrt(Is))
    return x, wr, (wg, wu, wd), shared


def _experts(wg, wu, wd):
    return [(wg[e], wu[e], wd[e]) for e in range(wg.shape[0])]


def test_single_expert_is_textbook_swiglu_mlp():
    rng = np.random.default_rng(11)
    x, wr, (wg, wu, wd), _ = _rand_layer(rng, 17, 24, 1, 40, 0)
    res = oracle.layer_forward(x, wr, _experts(wg, wu, wd), 1)
    F = torch.nn.functional
    xt = torch.from_numpy(x)
    ref = F.linear(F.silu(F.linear(xt, torch.from_numpy(wg[0]))) * F.linear(xt, torch.from_numpy(wu[0])),
                   torch.from_numpy(wd[0])).numpy()
    np.testing.assert_allclose(res["y"], ref, rtol=1e-12, atol=1e-13)


def _dense_mixture(x, wr, wg, wu, wd, shared, k, bias=None):
    """Every expert on every token, masked by the routing: y = sum_e M[t,e] E_e(x_t) + S(x_t)."""
    T, E = x.shape[0], wg.shape[0]
    logits = (x @ wr.T).astype(np.float32)
    ids, w = oracle.route(logits, k, bias=bias)
    M = np.zeros((T, E))
    for t in range(T):
        for j in range(k):
            M[t, ids[t, j]] += w[t, j]
    F = torch.nn.functional
    xt = torch.from_numpy(x)
    y = np.zeros_like(x)
    for e in range(E):
        out_e = F.linear(F.silu(F.linear(xt, torch.from_numpy(wg[e]))) * F.linear(xt, torch.from_numpy(wu[e])),
                         torch.from_numpy(wd[e])).numpy()
        y += M[:, e:e + 1] * out_e
    if shared is not None:
        sg, su, sd = (torch.from_numpy(a) for a in shared)
        y += F.linear(F.silu(F.linear(xt, sg)) * F.linear(xt, su), sd).numpy()
    return y


@pytest.mark.parametrize("T,D,E,k,I,Is", [(64, 32, 16, 2, 24, 24), (37, 16, 9, 9, 8, 0), (50, 8, 24, 5, 4, 16)])
def test_layer_matches_dense_mixture(T, D, E, k, I, Is):
    rng = np.random.default_rng(12 + T)
    x, wr, (wg, wu, wd), shared = _rand_layer(rng, T, D, E, I, Is)
    res = oracle.layer_forward(x, wr, _experts(wg, wu, wd), k, shared=shared)
    ref = _dense_mixture(x, wr, wg, wu, wd, shared, k)
    np.testing.assert_allclose(res["y"], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_layer_with_bias_matches_dense_mixture():
    rng = np.random.default_rng(13)
    x, wr, (wg, wu, wd), shared = _rand_layer(rng, 80, 16, 20, 8, 8)
    bias = np.linspace(2.0, -2.0, 20).astype(np.float32)
    bias[-3:] = -np.inf
    logits = (x @ wr.T).astype(np.float32)
    res = oracle.layer_forward(x, wr, _experts(wg, wu, wd), 4, shared=shared, bias=bias, logits=logits)
    assert res["counts"][-3:].tolist() == [0, 0, 0]
    ref = _dense_mixture(x, wr, wg, wu, wd, shared, 4, bias=bias)
    np.testing.assert_allclose(res["y"], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_worked_example_closed_form():
    ex = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    inp, exp_ = ex["inputs"], ex["expected"]
    a = {k_: np.array(v, dtype=np.float64) for k_, v in inp.items() if k_ != "top_k"}
    experts = _experts(a["w_gate"], a["w_up"], a["w_down"])
    res = oracle.layer_forward(a["x"], a["w_router"], experts, inp["top_k"],
                               shared=(a["shared_gate"], a["shared_up"], a["shared_down"]))
    assert res["ids"].tolist() == exp_["ids"]
    s = 1.0 / (1.0 + math.exp(-1.0))
    np.testing.assert_allclose(res["weights"], [[s, 1 - s], [0.5, 0.5]], rtol=1e-15)
    assert res["counts"].tolist() == exp_["counts"]
    assert res["offsets"].tolist() == exp_["offsets"]
    assert res["perm_token"].tolist() == exp_["perm_token"]
    assert res["inv_pos"].tolist() == exp_["inv_pos"]
    np.testing.assert_allclose(res["y"], exp_["y"], rtol=1e-14, atol=1e-15)


def test_zero_input_gives_zero_output():
    rng = np.random.default_rng(14)
    _, wr, (wg, wu, wd), shared = _rand_layer(rng, 1, 16, 8, 8, 8)
    x = np.zeros((5, 16))
    res = oracle.layer_forward(x, wr, _experts(wg, wu, wd), 3, shared=shared)
    assert (res["y"] == 0).all()
    assert (res["ids"] == np.arange(3)).all()          # all logits tie at 0


def test_down_projection_linearity():
    rng = np.random.default_rng(15)
    x, wr, (wg, wu, wd), _ = _rand_layer(rng, 40, 16, 8, 8, 0)
    y1 = oracle.layer_forward(x, wr, _experts(wg, wu, wd), 2)["y"]
    y2 = oracle.layer_forward(x, wr, _experts(wg, wu, 2.0 * wd), 2)["y"]
    np.testing.assert_array_equal(y2, 2.0 * y1)       # power-of-two scaling is exact


def test_expert_parallel_slices_sum_to_full_layer():
    rng = np.random.default_rng(16)
    x, wr, (wg, wu, wd), _ = _rand_layer(rng, 96, 16, 32, 8, 0)
    full = oracle.layer_forward(x, wr, _experts(wg, wu, wd), 4)
    total = np.zeros_like(x)
    for b in range(0, 32, 8):
        part = oracle.layer_from_routing(x, full["ids"], full["weights"],
                                         _experts(wg[b:b + 8], wu[b:b + 8], wd[b:b + 8]),
                                         expert_begin=b, n_local=8)
        total += part["y"]
    np.testing.assert_allclose(total, full["y"], rtol=1e-12, atol=1e-13)


def test_token_output_matches_layer_rows():
    rng = np.random.default_rng(17)
    x, wr, (wg, wu, wd), shared = _rand_layer(rng, 30, 16, 12, 8, 8)
    res = oracle.layer_forward(x, wr, _experts(wg, wu, wd), 3, shared=shared)
    for t in (0, 7, 29):
        y_t = oracle.token_output(x[t], res["ids"][t], res["weights"][t], _experts(wg, wu, wd), shared=shared)
        np.testing.assert_allclose(y_t, res["y"][t], rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------------------
# FP8 share
# ---------------------------------------------------------------------------

def _fp8_weights(rng, n, out_dim, in_dim):
    """E4M3 codes (via torch's cast) and fp32 per-output-channel scales."""
    z = rng.standard_normal((n, out_dim, in_dim)).astype(np.float32)
    amax = np.abs(z).max(axis=2, keepdims=True)
    codes = torch.from_numpy(np.clip(z * (448 / amax), -448, 448)).to(torch.float8_e4m3fn).double().numpy()
    scale = (amax[..., 0] / 448 / math.sqrt(in_dim)).astype(np.float32)
    return codes, scale


def test_fp8_share_with_single_intermediate_channel_is_exact_layer_on_dequantised_inputs():
    """With I = 1 each h row has one value, which the per-row quantiser maps to +-448 * s_h
    (exact up to fp32 rounding of the scale), so the fp8 share, quantising its float64 h
    (h_storage=None), must equal the exact layer evaluated on the dequantised x and weights:
    this pins where every scale enters."""
    rng = np.random.default_rng(18)
    T, D, E, k = 40, 32, 8, 3
    x = numerics.bf16_round(rng.standard_normal((T, D)).astype(np.float32))
    gq, gs = _fp8_weights(rng, E, 1, D)
    uq, us = _fp8_weights(rng, E, 1, D)
    dq, ds = _fp8_weights(rng, E, D, 1)
    ids, w = oracle.route(rng.standard_normal((T, E)).astype(np.float32), k)
    experts_q = [((gq[e], gs[e]), (uq[e], us[e]), (dq[e], ds[e])) for e in range(E)]
    got = oracle.layer_from_routing_fp8(x, ids, w, experts_q, h_storage=None)
    xq, sx = oracle.quantize_rows_e4m3(x)
    x_deq = xq * sx.astype(np.float64)[:, None]
    deq = [(gq[e] * gs[e][:, None], uq[e] * us[e][:, None], dq[e] * ds[e][:, None]) for e in range(E)]
    ref = oracle.layer_from_routing(x_deq, ids, w, deq)
    np.testing.assert_allclose(got["y"], ref["y"], rtol=0, atol=2e-6 * np.abs(ref["y"]).max())


def test_fp8_layer_shared_expert_runs_unquantised_on_x_with_weight_one():
    """The fp8 layer with a shared expert = its routed part (pinned above) + the shared
    expert of the exact bf16 layer evaluated on the unquantised x.  The shared-only term
    comes from the exact layer with all routing weights zero, so a shared expert applied
    to the quantised x, scaled, or dropped fails."""
    rng = np.random.default_rng(23)
    T, D, E, k, Is = 24, 32, 6, 2, 16
    x = numerics.bf16_round(rng.standard_normal((T, D)).astype(np.float32))
    gq, gs = _fp8_weights(rng, E, 1, D)
    uq, us = _fp8_weights(rng, E, 1, D)
    dq, ds = _fp8_weights(rng, E, D, 1)
    sh = tuple(numerics.bf16_round((rng.standard_normal(shape) / np.sqrt(shape[1])).astype(np.float32))
               for shape in ((Is, D), (Is, D), (D, Is)))
    ids, w = oracle.route(rng.standard_normal((T, E)).astype(np.float32), k)
    experts_q = [((gq[e], gs[e]), (uq[e], us[e]), (dq[e], ds[e])) for e in range(E)]
    got = oracle.layer_from_routing_fp8(x, ids, w, experts_q, shared=sh)["y"]
    routed = oracle.layer_from_routing_fp8(x, ids, w, experts_q)["y"]
    deq = [(gq[e] * gs[e][:, None], uq[e] * us[e][:, None], dq[e] * ds[e][:, None]) for e in range(E)]
    shared_only = oracle.layer_from_routing(x, ids, np.zeros_like(w), deq, shared=sh)["y"]
    assert np.abs(shared_only).max() > 0.1
    np.testing.assert_allclose(got, routed + shared_only, rtol=0, atol=1e-12 * np.abs(got).max())


def test_fp8_share_quantises_h_from_its_bf16_values():
    """By default h is stored as bf16 before its per-row quantisation: the h that enters the
    quantiser lies on the bf16 grid, within half a bf16 step of the float64 h (the step of its
    binade, 2**(e-7) for 2**e <= |h| < 2**(e+1), plus the binary32 rounding taken first), and
    the layer with h_storage=None (float64 h) differs from it; a dropped, truncating or
    wrong-grid rounding fails one of these."""
    rng = np.random.default_rng(31)
    T, D, E, k, I = 48, 64, 6, 2, 32
    x = numerics.bf16_round(rng.standard_normal((T, D)).astype(np.float32))
    gq, gs = _fp8_weights(rng, E, I, D)
    uq, us = _fp8_weights(rng, E, I, D)
    dq, ds = _fp8_weights(rng, E, D, I)
    ids, w = oracle.route(rng.standard_normal((T, E)).astype(np.float32), k)
    experts_q = [((gq[e], gs[e]), (uq[e], us[e]), (dq[e], ds[e])) for e in range(E)]
    got = oracle.layer_from_routing_fp8(x, ids, w, experts_q)
    raw = oracle.layer_from_routing_fp8(x, ids, w, experts_q, h_storage=None)
    h, h64 = got["h"], raw["h"]
    assert h.shape == (T * k, I)
    np.testing.assert_array_equal(numerics.bf16_round(h), h)
    _, ex = np.frexp(h)                                  # |h| = m * 2**ex, m in [0.5, 1)
    half_step = np.ldexp(1.0, ex - 9)                    # half of 2**((ex - 1) - 7)
    assert np.all(np.abs(h - h64) <= half_step * (1 + 2.0 ** -15))
    assert np.any(h != h64)
    assert not np.array_equal(got["y"], raw["y"])
    with pytest.raises(ValueError):
        oracle.layer_from_routing_fp8(x, ids, w, experts_q, h_storage="e4m3")


def test_fp8_share_close_to_exact_layer():
    """Quantisation moves y by a few percent at these small widths (each E4M3 operand carries
    up to 2**-4 relative error); a dropped or doubled scale would move it by O(1).  Where
    each scale enters is pinned exactly by the single-channel test above."""
    rng = np.random.default_rng(19)
    T, D, E, k, I = 64, 128, 8, 2, 64
    x = numerics.bf16_round(rng.standard_normal((T, D)).astype(np.float32))
    gq, gs = _fp8_weights(rng, E, I, D)
    uq, us = _fp8_weights(rng, E, I, D)
    dq, ds = _fp8_weights(rng, E, D, I)
    ids, w = oracle.route(rng.standard_normal((T, E)).astype(np.float32), k)
    experts_q = [((gq[e], gs[e]), (uq[e], us[e]), (dq[e], ds[e])) for e in range(E)]
    got = oracle.layer_from_routing_fp8(x, ids, w, experts_q, expert_begin=0, n_local=E)
    deq = [(gq[e] * gs[e][:, None], uq[e] * us[e][:, None], dq[e] * ds[e][:, None]) for e in range(E)]
    ref = oracle.layer_from_routing(x, ids, w, deq)
    err = np.abs(got["y"] - ref["y"]).max() / np.abs(ref["y"]).max()
    assert 1e-4 < err < 0.1
    # x codes are per-token and exact for the stored bf16 values
    q, s = oracle.quantize_rows_e4m3(x)
    np.testing.assert_array_equal(got["x_q"], q)
