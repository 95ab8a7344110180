"""The routed MoE FFN layer, step by step, in float64 NumPy.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The layer, as the pages state the problem:

* hidden size D, E = 512 small routed experts of intermediate size
  I = 1024, a router that keeps the top 10 experts per token through a
  softmax distribution, and one always-on shared expert
  ([PB] "The Architectural Constraints That Break Naive Sharding";
  [IM] "Por que esse modelo é difícil de servir"; [VN] "3. Sparse
  Mixture-of-Experts (MoE)");
* tokens are grouped by expert for the grouped GEMMs and "unpermuted"
  with a local reduction afterwards ([PB] "Three High-Leverage
  Optimizations", the SparseCore unpermutation row);
* under expert parallelism a device owns a contiguous slice of 64 of
  the 512 experts, receives the routing of all gathered tokens as one
  packed 32-bit blob of ids and weights, and produces partial sums that
  a reduce-scatter adds up ([PB] "Fusing Three Collectives Into Two";
  [IM] "O problema do sharding e a solução").

Readings taken where the pages are silent (the MoE formula on [VN] §3
breaks off after its colon):

* routing: softmax over all E keys, keep the k largest, renormalise the
  kept probabilities to sum to one (equal to a softmax over the k kept
  keys); selection compares the fp32 keys, larger first, and an equal key
  goes to the lower expert index; slot j holds the j-th selected expert;
* expert: SwiGLU, out = W_down (silu(W_gate x) * (W_up x)),
  silu(z) = z / (1 + exp(-z)); weights stored [out][in];
* shared expert: the same SwiGLU form, added with weight one (no gate);
* no capacity limit: every (token, slot) pair is computed.
"""

import numpy as np

from .numerics import bf16_round, f32_round, e4m3_round


# ---------------------------------------------------------------------------
# Router: logits, top-k, weights, packed blob
# ---------------------------------------------------------------------------

def router_logits(x, w_router):
    """Router projection logits[t, e] = sum_d x[t, d] * W_r[e, d].

    Exact float64 product sums of the stored values, rounded once to fp32
    (the pages note routing is sensitive to low-precision accumulation,
    [PB] "Roofline Validation", so the logits are kept in fp32).
    Returns float32 [T, E].
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w_router, dtype=np.float64)
    return (x @ w.T).astype(np.float32)


def route(logits, top_k, bias=None, renormalize=True):
    """Top-k routing over E experts from fp32 logits.

    key = fp32(logit + bias) (one fp32 add; bias is an optional [E]
    workload device that shifts expert popularity).  The k kept experts
    are the first k of a stable sort of the keys in descending order, so
    equal keys (including -0.0 vs +0.0) go to the lower expert index.
    Weights: softmax over all E keys in float64, then the kept entries
    divided by their sum when ``renormalize`` (the default), else the
    kept softmax entries as they are.

    Keys may be -inf (an expert that can never be chosen) as long as each
    token keeps at least k finite keys.  Returns (ids int32 [T, k],
    weights float64 [T, k]).
    """
    keys = np.asarray(logits, dtype=np.float32)
    if bias is not None:
        keys = (keys + np.asarray(bias, dtype=np.float32)[None, :]).astype(np.float32)
    T, E = keys.shape
    if not 1 <= top_k <= E:
        raise ValueError("top_k must be in [1, E]")
    order = np.argsort(-keys, axis=1, kind="stable")
    ids = order[:, :top_k]
    k64 = keys.astype(np.float64)
    kmax = k64.max(axis=1, keepdims=True)
    p = np.exp(k64 - kmax)
    p = p / p.sum(axis=1, keepdims=True)
    w = np.take_along_axis(p, ids, axis=1)
    if renormalize:
        w = w / w.sum(axis=1, keepdims=True)
    return ids.astype(np.int32), w


def pack_routing(ids, weights):
    """Pack ids and weights into one int32 blob of shape [T, 2, k].

    Plane 0 holds the expert ids, plane 1 the fp32 bit pattern of each
    weight ([PB] "Fusing Three Collectives Into Two": ids and weights of
    equal shape are stacked, bitcast and sent as one 32-bit array).
    Token-major, so blobs of several devices concatenate along tokens.
    """
    ids = np.asarray(ids, dtype=np.int32)
    w32 = np.ascontiguousarray(np.asarray(weights, dtype=np.float32))
    return np.stack([ids, w32.view(np.int32)], axis=1)


def unpack_routing(packed):
    """Inverse of :func:`pack_routing`: (ids int32 [T, k], weights float32 [T, k])."""
    packed = np.ascontiguousarray(np.asarray(packed, dtype=np.int32))
    return packed[:, 0, :].copy(), packed[:, 1, :].copy().view(np.float32)


# ---------------------------------------------------------------------------
# Permutation (grouping rows by expert) and its inverse
# ---------------------------------------------------------------------------

def permute(ids, expert_begin=0, n_local=None):
    """Group the (token, slot) pairs of the local experts by expert.

    The local experts are ids expert_begin .. expert_begin + n_local - 1;
    any other id (another device's expert, or an id out of range) is not
    local.  Over the token-major list of (t, j) pairs, the local pairs are
    stably sorted by expert: experts ascending, and (t, j) ascending
    within one expert.

    Returns
      counts     int64 [n_local]      rows of each local expert
      offsets    int64 [n_local + 1]  exclusive prefix sum; offsets[-1] = N_a
      perm_token int64 [N_a]          source token of each grouped row
      inv_pos    int64 [T, k]         grouped row of (t, j), or -1 if not local
    """
    ids = np.asarray(ids, dtype=np.int64)
    T, k = ids.shape
    if n_local is None:
        n_local = int(ids.max()) + 1 if ids.size else 0
    flat = ids.reshape(-1) - expert_begin
    local = (flat >= 0) & (flat < n_local)
    pairs = np.nonzero(local)[0]                       # ascending (t, j) order
    order = np.argsort(flat[pairs], kind="stable")
    grouped = pairs[order]
    counts = np.bincount(flat[pairs], minlength=n_local).astype(np.int64)
    offsets = np.zeros(n_local + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    perm_token = grouped // k
    inv_pos = np.full(T * k, -1, dtype=np.int64)
    inv_pos[grouped] = np.arange(grouped.size, dtype=np.int64)
    return counts, offsets, perm_token, inv_pos.reshape(T, k)


# ---------------------------------------------------------------------------
# Expert FFN and combine
# ---------------------------------------------------------------------------

def silu(z):
    """silu(z) = z * sigmoid(z) = z / (1 + exp(-z))."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_expert(x_rows, w_gate, w_up, w_down):
    """One expert on a block of rows: W_down (silu(W_gate x) * (W_up x)).

    x_rows [R, D]; w_gate, w_up [I, D]; w_down [D, I] (all [out][in]).
    Returns float64 [R, D].
    """
    x_rows = np.asarray(x_rows, dtype=np.float64)
    g = x_rows @ np.asarray(w_gate, dtype=np.float64).T
    u = x_rows @ np.asarray(w_up, dtype=np.float64).T
    h = silu(g) * u
    return h @ np.asarray(w_down, dtype=np.float64).T


def combine(out_rows, weights, inv_pos, shared_out=None):
    """Unpermute and reduce: y[t] = sum_j w[t, j] * out_rows[inv_pos[t, j]] (+ shared[t]).

    Slots whose expert is not local (inv_pos = -1) contribute nothing, so
    with a local slice the result is that slice's partial sum.
    """
    out_rows = np.asarray(out_rows, dtype=np.float64)
    weights = np.asarray(weights, dtype=np.float64)
    T, k = inv_pos.shape
    D = out_rows.shape[1] if out_rows.ndim == 2 else (shared_out.shape[1] if shared_out is not None else 0)
    y = np.zeros((T, D), dtype=np.float64)
    for j in range(k):
        rows = inv_pos[:, j]
        m = rows >= 0
        y[m] += weights[m, j][:, None] * out_rows[rows[m]]
    if shared_out is not None:
        y += np.asarray(shared_out, dtype=np.float64)
    return y


def _routed_rows(x, perm_token, offsets, experts):
    """Grouped expert evaluation: for each local expert, its rows in one block."""
    n_local = len(offsets) - 1
    D = x.shape[1]
    out = np.zeros((int(offsets[-1]), D), dtype=np.float64)
    for e in range(n_local):
        s, t = int(offsets[e]), int(offsets[e + 1])
        if s == t:
            continue                                   # empty group: nothing to do
        wg, wu, wd = experts[e]
        out[s:t] = swiglu_expert(x[perm_token[s:t]], wg, wu, wd)
    return out


def layer_from_routing(x, ids, weights, experts, *, shared=None, expert_begin=0, n_local=None):
    """Routed layer given the routing: permute -> grouped experts -> combine (+ shared).

    ``experts[e]`` for e in 0..n_local-1 returns (w_gate [I, D], w_up [I, D],
    w_down [D, I]) of local expert expert_begin + e (any indexable: an
    array, or a lazy loader).  ``shared`` is (w_gate, w_up, w_down) of the
    shared expert, or None.  Returns a dict with the permutation, the
    grouped expert outputs and y (float64 [T, D]).
    """
    x = np.asarray(x, dtype=np.float64)
    if n_local is None:
        n_local = len(experts)
    counts, offsets, perm_token, inv_pos = permute(ids, expert_begin, n_local)
    out_rows = _routed_rows(x, perm_token, offsets, experts)
    shared_out = swiglu_expert(x, *shared) if shared is not None else None
    y = combine(out_rows, weights, inv_pos, shared_out)
    return dict(counts=counts, offsets=offsets, perm_token=perm_token, inv_pos=inv_pos,
                out_rows=out_rows, shared_out=shared_out, y=y)


def layer_forward(x, w_router, experts, top_k, *, shared=None, bias=None, renormalize=True,
                  expert_begin=0, n_local=None, logits=None):
    """The whole layer: router -> route -> permute -> grouped experts -> combine.

    ``logits`` (fp32 [T, E]) may be given to route from exactly the same
    logits as another implementation; otherwise they come from
    :func:`router_logits`.  Returns the dict of :func:`layer_from_routing`
    plus logits, ids and weights.
    """
    if logits is None:
        logits = router_logits(x, w_router)
    ids, w = route(logits, top_k, bias=bias, renormalize=renormalize)
    res = layer_from_routing(x, ids, w, experts, shared=shared,
                             expert_begin=expert_begin, n_local=n_local)
    res.update(logits=np.asarray(logits, dtype=np.float32), ids=ids, weights=w)
    return res


def token_output(x_t, ids_t, w_t, experts, *, shared=None, expert_begin=0, n_local=None):
    """y for one token straight from the definition: sum_j w_j E_{id_j}(x) + S(x).

    Used to check sampled tokens of a full-size layer without evaluating
    the others.  Non-local ids contribute nothing.
    """
    x_t = np.asarray(x_t, dtype=np.float64)[None, :]
    if n_local is None:
        n_local = len(experts)
    y = np.zeros(x_t.shape[1], dtype=np.float64)
    for e, w in zip(np.asarray(ids_t).tolist(), np.asarray(w_t, dtype=np.float64).tolist()):
        le = e - expert_begin
        if 0 <= le < n_local:
            y += w * swiglu_expert(x_t, *experts[le])[0]
    if shared is not None:
        y += swiglu_expert(x_t, *shared)[0]
    return y


# ---------------------------------------------------------------------------
# FP8 (E4M3) variant for one device's expert-parallel share
# ---------------------------------------------------------------------------

def quantize_rows_e4m3(a):
    """Per-row E4M3 quantisation with an fp32 scale.

    Reading of "FP8 scaling blocks" ([PB] "Roofline Validation") for the
    activations: one block per row.  The row is taken in fp32; its scale
    is s = fp32(amax / 448) (s = 1 for an all-zero row); each value is
    divided by s in fp32 and rounded to E4M3 (nearest-even, saturating).
    Returns (q float64 [R, C] on the E4M3 grid, s float32 [R]); the
    dequantised row is q * s.
    """
    a32 = np.asarray(a, dtype=np.float64).astype(np.float32)
    amax = np.abs(a32).max(axis=1) if a32.shape[1] else np.zeros(a32.shape[0], np.float32)
    s = (amax / np.float32(448.0)).astype(np.float32)
    s = np.where(amax == 0, np.float32(1.0), s).astype(np.float32)
    scaled = (a32 / s[:, None]).astype(np.float32)
    return e4m3_round(scaled.astype(np.float64)), s


def layer_from_routing_fp8(x, ids, weights, experts_q, *, shared=None, expert_begin=0, n_local=None,
                           h_storage="bf16"):
    """The routed layer with e4m3 expert weights and per-output-channel scales.

    ``experts_q[e]`` returns ((g_q, g_s), (u_q, u_s), (d_q, d_s)): codes as
    float64 values on the E4M3 grid ([I, D], [I, D], [D, I]) and fp32
    scales per output channel ([I], [I], [D]).  Steps:

    1. quantise each token's activations (per-token scale);
    2. permute as in :func:`permute`;
    3. per expert: g = (x_q W_gq^T) s_x s_g, u likewise, h = silu(g) * u
       in float64;
    4. store h in the activation type (bfloat16: ``h_storage="bf16"``) and
       quantise the stored rows per grouped row, so that h's codes are
       decided from the values the layer keeps, as x's are from the given
       bf16 x; out = (h_q W_dq^T) s_h s_d.  ``h_storage=None`` quantises
       the float64 h itself (what the pin of each scale's place uses);
    5. combine with the routing weights, plus the shared expert when
       ``shared`` = (w_gate, w_up, w_down) is given.  The pages give the
       routed experts' fp8 storage only; the shared expert keeps the
       activation precision (its exact float64 image here, unquantised).
       One device's expert-parallel share passes no shared expert: its
       partial sums go to a reduce-scatter and the shared expert is added
       once per token by the device that owns the token.
    """
    if h_storage not in ("bf16", None):
        raise ValueError(f"h_storage must be 'bf16' or None, not {h_storage!r}")
    x = np.asarray(x, dtype=np.float64)
    if n_local is None:
        n_local = len(experts_q)
    xq, sx = quantize_rows_e4m3(x)
    counts, offsets, perm_token, inv_pos = permute(ids, expert_begin, n_local)
    D = x.shape[1]
    out = np.zeros((int(offsets[-1]), D), dtype=np.float64)
    h_rows = None
    for e in range(n_local):
        s, t = int(offsets[e]), int(offsets[e + 1])
        if s == t:
            continue
        (gq, gs), (uq, us), (dq, ds) = experts_q[e]
        rows = perm_token[s:t]
        xs = sx[rows].astype(np.float64)[:, None]
        g = (xq[rows] @ np.asarray(gq, np.float64).T) * xs * np.asarray(gs, np.float64)[None, :]
        u = (xq[rows] @ np.asarray(uq, np.float64).T) * xs * np.asarray(us, np.float64)[None, :]
        h = silu(g) * u
        if h_storage == "bf16":
            h = bf16_round(h)
        if h_rows is None:
            h_rows = np.zeros((int(offsets[-1]), h.shape[1]), dtype=np.float64)
        h_rows[s:t] = h
        hq, hs = quantize_rows_e4m3(h)
        out[s:t] = (hq @ np.asarray(dq, np.float64).T) * hs.astype(np.float64)[:, None] \
            * np.asarray(ds, np.float64)[None, :]
    shared_out = swiglu_expert(x, *shared) if shared is not None else None
    y = combine(out, weights, inv_pos, shared_out)
    return dict(counts=counts, offsets=offsets, perm_token=perm_token, inv_pos=inv_pos,
                x_q=xq, x_scale=sx, h=h_rows, out_rows=out, shared_out=shared_out, y=y)
