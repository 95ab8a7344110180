// C ABI of the MoE layer: argument validation, workspace layout, launch sequences.
// Every check happens on the host before the first launch; the library never
// allocates, frees or synchronises.
#include <stddef.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "moe.h"
#include "common.hpp"
#include "kernels.hpp"

using namespace moe;

namespace {

thread_local int g_last_hip_error = 0;

size_t align_up(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

int act_size(int dt) { return dt == MOE_F32 ? 4 : 2; }
int out_size(int dt) { return dt == MOE_F32 ? 4 : 2; }
int w_el(const moe_dims& d) { return d.w_dtype; }
int h_el(const moe_dims& d) { return d.act_dtype == MOE_F32 ? EL_F32 : EL_BF16; }

int check_dims(const moe_dims* d) {
  if (!d) return MOE_ERR_NULL_ARG;
  if (d->T < 0 || d->D < 1 || d->E < 1 || d->I < 1 || d->top_k < 1 || d->top_k > d->E) return MOE_ERR_BAD_DIMS;
  if (d->I_shared < 0 || d->expert_begin < 0 || d->n_local < 1 ||
      static_cast<int64_t>(d->expert_begin) + d->n_local > d->E)
    return MOE_ERR_BAD_DIMS;
  if (d->renormalize != 0 && d->renormalize != 1) return MOE_ERR_BAD_DIMS;
  if (d->weight_layout != MOE_LAYOUT_ROWS && d->weight_layout != MOE_LAYOUT_PACKED) return MOE_ERR_BAD_DIMS;
  if (d->top_k > 32 || d->E > 1024 || d->n_local > kMaxLocalExperts) return MOE_ERR_UNSUPPORTED;
  if (d->D % 64 || d->I % 64 || d->I_shared % 64) return MOE_ERR_UNSUPPORTED;
  const bool f32 = d->act_dtype == MOE_F32 && d->w_dtype == MOE_F32 && d->out_dtype == MOE_F32;
  const bool bf16 = d->act_dtype == MOE_BF16 && (d->w_dtype == MOE_BF16 || d->w_dtype == MOE_E4M3) &&
                    (d->out_dtype == MOE_BF16 || d->out_dtype == MOE_F32);
  if (!f32 && !bf16) return MOE_ERR_UNSUPPORTED;
  // every row index and byte offset below fits the kernels' integer types
  const int64_t tk = static_cast<int64_t>(d->T) * d->top_k;
  if (tk > (1ll << 30) || static_cast<int64_t>(d->T) * d->E > (1ll << 31) - 1) return MOE_ERR_UNSUPPORTED;
  // one expert's (and the router's) weight matrix is addressed with 32-bit offsets
  const int64_t wsz = d->w_dtype == MOE_F32 ? 4 : d->w_dtype == MOE_BF16 ? 2 : 1;
  const int64_t lim = 1ll << 31;
  if (static_cast<int64_t>(d->I) * d->D * wsz >= lim ||
      static_cast<int64_t>(d->I_shared) * d->D * act_size(d->act_dtype) >= lim ||
      static_cast<int64_t>(d->E) * d->D * act_size(d->act_dtype) >= lim)
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// Router projection shape: 256-row tiles once there are enough tokens for each W_r byte
// to feed 256 of them (and x fits the tile shape's 32-bit offsets); 32-row streaming
// tiles below that.
int router_shape(const moe_dims& d) {
  const int64_t x_bytes = static_cast<int64_t>(d.T) * d.D * act_size(d.act_dtype);
  return d.T >= 2048 && x_bytes < (1ll << 31) ? kShapeTile256 : kShapeStream32;
}

// K splits of the router projection (partial sums added in order by the route kernel):
// enough workgroups to cover the chip, at most 256 tiles in the streaming shape (one per
// CU: at 512 tokens and 512 experts four partial sums, where eight or two made the
// routing stage slower) and at least 256 (with at most 4 partial products) in the tile
// shape.
int router_splits(const moe_dims& d) {
  const int shape = router_shape(d);
  const int row_bytes = d.D * act_size(d.act_dtype);
  const int kblk = shape == kShapeTile256 ? 128 : 512;  // bytes per K block of the shape
  if (row_bytes % kblk) return 1;
  const int blocks = row_bytes / kblk;
  const int bm = gemm_bm(shape), bn = gemm_bn(false, shape, d.act_dtype, false);
  const int64_t tiles = static_cast<int64_t>((d.T + bm - 1) / bm) * ((d.E + bn - 1) / bn);
  int s = 1;
  if (shape == kShapeTile256) {
    while (s < 4 && tiles * s < 256 && s * 2 <= blocks && blocks % (s * 2) == 0) s *= 2;
  } else {
    while (s * 2 <= blocks && blocks % (s * 2) == 0 && tiles * s * 2 <= 256) s *= 2;
  }
  return s;
}

struct Layout {
  size_t err, logits, logits_part, packed, hist, base, rank, bad, counts, offsets, tp_a, tp_b, perm_token, inv_pos;
  size_t cand_key, cand_id, cand_stats;
  size_t xq, sx, h, h_sh, hq, sh, out_rows, total;
};

Layout layout(const moe_dims& d) {
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align_up(bytes);
    return o;
  };
  const size_t T = d.T, tk = static_cast<size_t>(d.T) * d.top_k, nl = d.n_local;
  const size_t U = perm_units(d.T, d.top_k);
  const bool fp8 = d.w_dtype == MOE_E4M3;
  const size_t hs = act_size(d.act_dtype), os = out_size(d.out_dtype);
  L.err = take(4);  // MOE_WS_ERROR_OFFSET: first word of the workspace
  L.logits = take(T * d.E * 4);
  const int rs = router_splits(d);
  L.logits_part = take(rs > 1 ? static_cast<size_t>(rs) * T * d.E * 4 : 0);
  L.packed = take(tk * 2 * 4);
  const size_t ns = router_fused_slices(d.T, d.E);
  L.cand_key = take(T * ns * d.top_k * 4);
  L.cand_id = take(T * ns * d.top_k * 4);
  L.cand_stats = take(T * ns * 8);
  L.hist = take(nl * U * 4);
  L.base = take(nl * U * 4);
  L.rank = take(tk * 4);
  L.bad = take(U * 4);
  L.counts = take(nl * 4);
  L.offsets = take((nl + 1) * 4);
  L.tp_a = take((nl + 1) * 4);
  L.tp_b = take((nl + 1) * 4);
  L.perm_token = take(tk * 4);
  L.inv_pos = take(tk * 4);
  L.xq = take(fp8 ? T * d.D : 0);
  L.sx = take(fp8 ? T * 4 : 0);
  L.h = take(tk * d.I * hs);
  L.h_sh = take(T * d.I_shared * hs);
  L.hq = take(fp8 ? tk * d.I : 0);
  L.sh = take(fp8 ? tk * 4 : 0);
  L.out_rows = take(tk * d.D * os);
  L.total = off;
  return L;
}

template <typename P> P* at(void* ws, size_t off) { return reinterpret_cast<P*>(static_cast<uint8_t*>(ws) + off); }

int hip_status(hipError_t e) {
  if (e == hipSuccess) return MOE_OK;
  g_last_hip_error = static_cast<int>(e);
  return MOE_ERR_HIP;
}

#define MOE_TRY(expr)                        \
  do {                                       \
    const int _s = hip_status(expr);         \
    if (_s != MOE_OK) return _s;             \
  } while (0)

// Shape of the grouped expert GEMMs: the average routed rows per expert decides.  The
// tile shape addresses its operands with 32-bit offsets; batches whose operands do not
// fit below 2 GiB take the 32-row streaming shape instead.  gathered: the gate/up A
// operand is x ([T][D], read through perm) rather than grouped rows ([T * top_k][D]).
int expert_shape(const moe_dims& d, bool gathered) {
  const double avg = static_cast<double>(d.T) * d.top_k / d.E;
  if (avg <= 16.0) return kShapeStream16;
  if (avg <= 32.0) return kShapeStream32;
  const int64_t lim = 1ll << 31, tk = static_cast<int64_t>(d.T) * d.top_k;
  const int64_t ea = act_size(d.act_dtype);
  const int64_t ih = std::max(d.I, d.I_shared);
  const bool fits = (gathered ? d.T : tk) * d.D * ea < lim && tk * d.I * 4 < lim &&
                    static_cast<int64_t>(d.T) * d.I_shared * 4 < lim && static_cast<int64_t>(d.T) * d.D * ea < lim &&
                    ih * d.D * 4 < lim;
  return fits ? kShapeTile256 : kShapeStream32;
}

int routed_tile_bound(int rows_total, int n_groups, int bm, int n, int bn) {
  const int64_t mt = (static_cast<int64_t>(rows_total) + static_cast<int64_t>(n_groups) * (bm - 1)) / bm;
  return static_cast<int>(mt * ((n + bn - 1) / bn));
}

GemmProblem problem(const void* a, const int32_t* perm, const float* a_scale, int lda, const int32_t* offsets,
                    const int32_t* tile_prefix, int n_groups, int rows, const void* w0, const void* w1,
                    const float* s0, const float* s1, long long w_stride, void* out, int ldo, int N, int K) {
  GemmProblem p;
  p.a = a; p.perm = perm; p.a_scale = a_scale; p.lda = lda;
  p.offsets = offsets; p.tile_prefix = tile_prefix; p.n_groups = n_groups; p.rows = rows;
  p.w0 = w0; p.w1 = w1; p.s0 = s0; p.s1 = s1; p.w_stride = w_stride;
  p.out = out; p.ldo = ldo; p.N = N; p.K = K;
  p.k_splits = 1; p.out_split_stride = 0;
  p.comb_rows = nullptr; p.comb_packed = nullptr; p.comb_inv = nullptr; p.comb_k = 0;
  return p;
}

// The fused router (projection and per-slice top-k, then an exact merge) addresses x and
// W_r with 32-bit offsets.
bool fused_router_fits(const moe_dims& d) {
  const int64_t es = act_size(d.act_dtype);
  return static_cast<int64_t>(d.T) * d.D * es < (1ll << 31) && static_cast<int64_t>(d.E) * d.D * es < (1ll << 31);
}

int route_fused(const moe_dims& d, const Layout& L, void* ws, const void* x, const void* w_router, float* logits,
                const float* bias, int32_t* packed, hipStream_t s) {
  return hip_status(launch_router_topk(d.act_dtype, x, w_router, bias, d.T, d.D, d.E, d.top_k, d.renormalize, logits,
                                       packed, at<float>(ws, L.cand_key), at<int32_t>(ws, L.cand_id),
                                       at<float2>(ws, L.cand_stats), s));
}

// Router projection + top-k.  parts: scratch for split-K partial products (NULL: no split).
int route_tokens(const moe_dims& d, const void* x, const void* w_router, float* logits, float* parts,
                 const float* bias, int32_t* packed, hipStream_t s) {
  if (x) {
    const int splits = parts ? router_splits(d) : 1;
    GemmProblem p = problem(x, nullptr, nullptr, d.D, nullptr, nullptr, 1, d.T, w_router, nullptr, nullptr, nullptr,
                            0, splits > 1 ? parts : logits, d.E, d.E, d.D);
    p.k_splits = splits;
    p.out_split_stride = static_cast<long long>(d.T) * d.E;
    const int shape = router_shape(d);
    const int bm = gemm_bm(shape), bn = gemm_bn(false, shape, d.act_dtype, false);
    const int tiles = ((d.T + bm - 1) / bm) * ((d.E + bn - 1) / bn) * splits;
    MOE_TRY(launch_gemm(d.act_dtype, EL_F32, false, shape, false, p, tiles, s));
    return hip_status(launch_route(parts, splits, logits, bias, d.T, d.E, d.top_k, d.renormalize, packed, s));
  }
  return hip_status(launch_route(nullptr, 1, logits, bias, d.T, d.E, d.top_k, d.renormalize, packed, s));
}

// gate/up -> h (+ quantise) -> down for the routed groups, then the optional shared
// expert in launches of its own, whose down projection also does the unpermute-combine:
// y[t] = sum_j w[t][j] * out_rows[inv[t][j]] + shared(x_t).
int experts_forward(const moe_dims& d, void* ws, const Layout& L, const void* a_rows, const float* a_scale,
                    const int32_t* perm, const int32_t* offsets, const void* w_gate, const void* w_up,
                    const void* w_down, const float* s_gate, const float* s_up, const float* s_down,
                    void* out_rows, const void* x_shared, const void* sh_gate, const void* sh_up,
                    const void* sh_down, void* y, const int32_t* comb_packed, const int32_t* comb_inv,
                    bool have_tile_prefix, hipEvent_t ev_gate_up, hipEvent_t ev_down, hipStream_t s) {
  const int shape = expert_shape(d, perm != nullptr);
  const bool packed = d.weight_layout == MOE_LAYOUT_PACKED;
  const int bm = gemm_bm(shape);
  const int bn_gu = gemm_bn(true, shape, w_el(d), packed), bn_dn = gemm_bn(false, shape, w_el(d), packed);
  const int tk = d.T * d.top_k;
  const bool fp8 = d.w_dtype == MOE_E4M3;
  int32_t* tp_a = at<int32_t>(ws, L.tp_a);
  int32_t* tp_b = at<int32_t>(ws, L.tp_b);
  void* h = at<void>(ws, L.h);
  void* h_sh = at<void>(ws, L.h_sh);
  const int32_t* n_rows_dev = offsets + d.n_local;
  const int hel = h_el(d);
  const bool shared = d.I_shared > 0 && sh_gate;

  if (!have_tile_prefix) MOE_TRY(launch_tile_prefix(offsets, d.n_local, bm, bm, tp_a, tp_b, s));

  // gate/up with the fused SwiGLU epilogue
  const GemmProblem g0 = problem(a_rows, perm, a_scale, d.D, offsets, tp_a, d.n_local, 0, w_gate, w_up, s_gate, s_up,
                                 static_cast<long long>(d.I) * d.D, h, d.I, d.I, d.D);
  const int tiles_gu = routed_tile_bound(tk, d.n_local, bm, d.I, bn_gu);
  MOE_TRY(launch_gemm(w_el(d), hel, true, shape, packed, g0, tiles_gu, s));
  if (ev_gate_up) MOE_TRY(hipEventRecord(ev_gate_up, s));

  // down projection of every grouped row
  const void* h_in = h;
  const float* h_scale = nullptr;
  if (fp8) {
    void* hq = at<void>(ws, L.hq);
    float* sh = at<float>(ws, L.sh);
    MOE_TRY(launch_quant_rows(EL_BF16, h, tk, n_rows_dev, d.I, hq, sh, s));
    h_in = hq;
    h_scale = sh;
  }
  const GemmProblem d0 = problem(h_in, nullptr, h_scale, d.I, offsets, tp_b, d.n_local, 0, w_down, nullptr, s_down,
                                 nullptr, static_cast<long long>(d.D) * d.I, out_rows, d.D, d.D, d.I);
  const int tiles_dn = routed_tile_bound(tk, d.n_local, bm, d.D, bn_dn);
  const int oel = d.out_dtype;
  MOE_TRY(launch_gemm(w_el(d), oel, false, shape, packed, d0, tiles_dn, s));
  if (ev_down) MOE_TRY(hipEventRecord(ev_down, s));

  // The shared expert runs in launches of its own: as a second problem of the routed
  // launches its tiles (all full, and last in the launch order) landed on one XCD.  Where
  // the routed GEMMs stream 16-row tiles it takes 32-row ones: all T rows read the same
  // weights, and taller tiles halve those re-reads.
  if (shared) {
    const int sh_shape = shape == kShapeStream16 ? kShapeStream32 : shape;
    const int sh_bm = gemm_bm(sh_shape);
    const int bn_g = gemm_bn(true, sh_shape, d.act_dtype, packed);
    const int bn_d = gemm_bn(false, sh_shape, d.act_dtype, packed);
    const GemmProblem gs = problem(x_shared, nullptr, nullptr, d.D, nullptr, nullptr, 1, d.T, sh_gate, sh_up, nullptr,
                                   nullptr, 0, h_sh, d.I_shared, d.I_shared, d.D);
    MOE_TRY(launch_gemm(d.act_dtype, hel, true, sh_shape, packed, gs,
                        ((d.T + sh_bm - 1) / sh_bm) * ((d.I_shared + bn_g - 1) / bn_g), s));
    GemmProblem ds = problem(h_sh, nullptr, nullptr, d.I_shared, nullptr, nullptr, 1, d.T, sh_down, nullptr,
                             nullptr, nullptr, 0, y, d.D, d.D, d.I_shared);
    ds.comb_rows = out_rows;
    ds.comb_packed = comb_packed;
    ds.comb_inv = comb_inv;
    ds.comb_k = d.top_k;
    MOE_TRY(launch_gemm_combine(d.act_dtype, oel, sh_shape, packed, ds,
                                ((d.T + sh_bm - 1) / sh_bm) * ((d.D + bn_d - 1) / bn_d), s));
  }
  return MOE_OK;
}

// Static scratch of moe_layer_forward_noalloc.  In host code `scratch` names a host-side
// stand-in, not device memory: kernels only ever see the device address that
// hipGetSymbolAddress returns for the current device, looked up once per device.
__device__ __align__(256) uint8_t scratch[MOE_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

int static_scratch(void** out) {
  int dev = 0;
  MOE_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    MOE_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

size_t moe_workspace_bytes(const moe_dims* dims) {
  if (check_dims(dims) != MOE_OK) return 0;
  return layout(*dims).total;
}

int moe_route(const moe_dims* dims, const void* x, const void* w_router, float* logits, const float* logit_bias,
              int32_t* packed, void* ws, size_t ws_bytes, void* stream) {
  int st = check_dims(dims);
  if (st != MOE_OK) return st;
  const moe_dims& d = *dims;
  if (!logits || !packed) return MOE_ERR_NULL_ARG;
  if ((x == nullptr) != (w_router == nullptr)) return MOE_ERR_NULL_ARG;
  const Layout L = layout(d);
  if (ws && ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (d.T == 0) return MOE_OK;
  return route_tokens(d, x, w_router, logits, ws ? at<float>(ws, L.logits_part) : nullptr, logit_bias, packed,
                      static_cast<hipStream_t>(stream));
}

int moe_route_fused(const moe_dims* dims, const void* x, const void* w_router, float* logits, const float* logit_bias,
                    int32_t* packed, void* ws, size_t ws_bytes, void* stream) {
  int st = check_dims(dims);
  if (st != MOE_OK) return st;
  const moe_dims& d = *dims;
  if (!x || !w_router || !packed || !ws) return MOE_ERR_NULL_ARG;
  if (!fused_router_fits(d)) return MOE_ERR_UNSUPPORTED;
  const Layout L = layout(d);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (d.T == 0) return MOE_OK;
  return route_fused(d, L, ws, x, w_router, logits, logit_bias, packed, static_cast<hipStream_t>(stream));
}

int moe_permute(const moe_dims* dims, const int32_t* packed, int32_t* counts, int32_t* offsets, int32_t* perm_token,
                int32_t* inv_pos, const void* x, void* x_perm, float* x_perm_scale, void* ws, size_t ws_bytes,
                void* stream) {
  int st = check_dims(dims);
  if (st != MOE_OK) return st;
  const moe_dims& d = *dims;
  if (!packed || !counts || !offsets || !perm_token || !inv_pos || !ws) return MOE_ERR_NULL_ARG;
  if ((x == nullptr) != (x_perm == nullptr)) return MOE_ERR_NULL_ARG;
  const bool fp8 = d.w_dtype == MOE_E4M3;
  if (x && fp8 && !x_perm_scale) return MOE_ERR_NULL_ARG;
  const Layout L = layout(d);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (d.T == 0) return MOE_OK;
  const int bm = gemm_bm(expert_shape(d, true));
  // e4m3: x is quantised per token by the grouping launches, as in the layer call
  const bool quant = x && fp8;
  MOE_TRY(launch_permute(packed, d.T, d.top_k, d.E, d.expert_begin, d.n_local, at<int32_t>(ws, L.hist),
                         at<int32_t>(ws, L.base), at<int32_t>(ws, L.rank), at<int32_t>(ws, L.bad), counts, offsets,
                         perm_token, inv_pos, bm, bm, at<int32_t>(ws, L.tp_a), at<int32_t>(ws, L.tp_b),
                         at<int32_t>(ws, L.err), s, quant ? x : nullptr, d.D, quant ? at<void>(ws, L.xq) : nullptr,
                         quant ? at<float>(ws, L.sx) : nullptr));
  if (x) {
    const int tk = d.T * d.top_k;
    if (fp8) {
      MOE_TRY(launch_gather_rows(at<void>(ws, L.xq), at<float>(ws, L.sx), perm_token, offsets + d.n_local, tk, d.D,
                                 x_perm, x_perm_scale, s));
    } else {
      MOE_TRY(launch_gather_rows(x, nullptr, perm_token, offsets + d.n_local, tk, d.D * act_size(d.act_dtype), x_perm,
                                 nullptr, s));
    }
  }
  return MOE_OK;
}

int moe_grouped_ffn(const moe_dims* dims, const void* a_rows, const float* a_scale, const int32_t* perm_token,
                    const int32_t* offsets, const void* w_gate, const void* w_up, const void* w_down,
                    const float* s_gate, const float* s_up, const float* s_down, void* out_rows, void* ws,
                    size_t ws_bytes, void* stream) {
  int st = check_dims(dims);
  if (st != MOE_OK) return st;
  const moe_dims& d = *dims;
  if (!a_rows || !offsets || !w_gate || !w_up || !w_down || !out_rows || !ws) return MOE_ERR_NULL_ARG;
  const bool fp8 = d.w_dtype == MOE_E4M3;
  if (fp8 && (!a_scale || !s_gate || !s_up || !s_down)) return MOE_ERR_NULL_ARG;
  const Layout L = layout(d);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (d.T == 0) return MOE_OK;
  return experts_forward(d, ws, L, a_rows, a_scale, perm_token, offsets, w_gate, w_up, w_down, s_gate, s_up, s_down,
                         out_rows, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, false, nullptr,
                         nullptr, static_cast<hipStream_t>(stream));
}

int moe_unpermute_combine(const moe_dims* dims, const void* out_rows, const int32_t* packed, const int32_t* inv_pos,
                          const void* shared_out, void* y, void* stream) {
  int st = check_dims(dims);
  if (st != MOE_OK) return st;
  const moe_dims& d = *dims;
  if (!out_rows || !packed || !inv_pos || !y) return MOE_ERR_NULL_ARG;
  if (d.T == 0) return MOE_OK;
  return hip_status(launch_combine(d.out_dtype, out_rows, packed, inv_pos, shared_out, d.T, d.D, d.top_k, y,
                                   static_cast<hipStream_t>(stream)));
}

int moe_layer_forward(const moe_dims* dims, const moe_weights* w, const void* x, const int32_t* packed_in,
                      const float* logit_bias, void* y, float* logits_out, int32_t* packed_out, void* ws,
                      size_t ws_bytes, void* const* stage_events, void* stream) {
  int st = check_dims(dims);
  if (st != MOE_OK) return st;
  const moe_dims& d = *dims;
  if (!w || !x || !y || !ws) return MOE_ERR_NULL_ARG;
  if (!w->w_gate || !w->w_up || !w->w_down) return MOE_ERR_NULL_ARG;
  if (!packed_in && !w->w_router) return MOE_ERR_NULL_ARG;
  const bool fp8 = d.w_dtype == MOE_E4M3;
  if (fp8 && (!w->s_gate || !w->s_up || !w->s_down)) return MOE_ERR_NULL_ARG;
  if (d.I_shared > 0 && (!w->sh_gate || !w->sh_up || !w->sh_down)) return MOE_ERR_NULL_ARG;
  const Layout L = layout(d);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (d.T == 0) return MOE_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto mark = [&](int i) -> hipError_t {
    return stage_events ? hipEventRecord(static_cast<hipEvent_t>(stage_events[i]), s) : hipSuccess;
  };
  MOE_TRY(mark(0));

  // 1. routing
  const int32_t* packed = packed_in;
  if (!packed_in) {
    float* logits = logits_out ? logits_out : at<float>(ws, L.logits);
    int32_t* pk = packed_out ? packed_out : at<int32_t>(ws, L.packed);
    st = route_tokens(d, x, w->w_router, logits, at<float>(ws, L.logits_part), logit_bias, pk, s);
    if (st != MOE_OK) return st;
    packed = pk;
  } else if (packed_out) {
    MOE_TRY(hipMemcpyAsync(packed_out, packed_in, static_cast<size_t>(d.T) * 2 * d.top_k * 4,
                           hipMemcpyDeviceToDevice, s));
  }

  MOE_TRY(mark(1));

  // 2. grouping by expert (and the tile schedule of both grouped GEMMs)
  int32_t* counts = at<int32_t>(ws, L.counts);
  int32_t* offsets = at<int32_t>(ws, L.offsets);
  int32_t* perm = at<int32_t>(ws, L.perm_token);
  int32_t* inv = at<int32_t>(ws, L.inv_pos);
  const int bm = gemm_bm(expert_shape(d, true));
  // with e4m3 experts the grouping launches also quantise x per token
  MOE_TRY(launch_permute(packed, d.T, d.top_k, d.E, d.expert_begin, d.n_local, at<int32_t>(ws, L.hist),
                         at<int32_t>(ws, L.base), at<int32_t>(ws, L.rank), at<int32_t>(ws, L.bad), counts, offsets,
                         perm, inv, bm, bm, at<int32_t>(ws, L.tp_a), at<int32_t>(ws, L.tp_b), at<int32_t>(ws, L.err),
                         s, fp8 ? x : nullptr, d.D, fp8 ? at<void>(ws, L.xq) : nullptr,
                         fp8 ? at<float>(ws, L.sx) : nullptr));
  const void* a_rows = fp8 ? at<void>(ws, L.xq) : x;
  const float* a_scale = fp8 ? at<float>(ws, L.sx) : nullptr;
  MOE_TRY(mark(2));

  // 3. experts; with a shared expert its down projection also does step 4 (the unpermute-
  // combine) in its epilogue and writes y
  void* out_rows = at<void>(ws, L.out_rows);
  const bool shared = d.I_shared > 0;
  st = experts_forward(d, ws, L, a_rows, a_scale, perm, offsets, w->w_gate, w->w_up, w->w_down, w->s_gate, w->s_up,
                       w->s_down, out_rows, x, shared ? w->sh_gate : nullptr, w->sh_up, w->sh_down, y, packed, inv,
                       true, stage_events ? static_cast<hipEvent_t>(stage_events[3]) : nullptr,
                       stage_events ? static_cast<hipEvent_t>(stage_events[4]) : nullptr, s);
  if (st != MOE_OK) return st;
  MOE_TRY(mark(5));

  // 4. unpermute + weighted combine (no shared expert: partial sums of the routed slots only)
  if (!shared) MOE_TRY(launch_combine(d.out_dtype, out_rows, packed, inv, nullptr, d.T, d.D, d.top_k, y, s));
  return hip_status(mark(6));
}

int moe_layer_forward_noalloc(const moe_dims* dims, const moe_weights* w, const void* x, const int32_t* packed_in,
                              const float* logit_bias, void* y, float* logits_out, int32_t* packed_out,
                              int32_t* bad_ids, void* const* stage_events, void* stream) {
  const int st = check_dims(dims);
  if (st != MOE_OK) return st;
  const size_t need = layout(*dims).total;
  if (need > MOE_STATIC_SCRATCH_BYTES) return MOE_ERR_SCRATCH_LIMIT;
  if (dims->T == 0) return MOE_OK;
  void* ws = nullptr;
  const int sst = static_scratch(&ws);
  if (sst != MOE_OK) return sst;
  const int r = moe_layer_forward(dims, w, x, packed_in, logit_bias, y, logits_out, packed_out, ws,
                                  MOE_STATIC_SCRATCH_BYTES, stage_events, stream);
  if (r != MOE_OK || !bad_ids) return r;
  return hip_status(hipMemcpyAsync(bad_ids, static_cast<uint8_t*>(ws) + MOE_WS_ERROR_OFFSET, sizeof(int32_t),
                                   hipMemcpyDeviceToDevice, static_cast<hipStream_t>(stream)));
}

size_t moe_audit_workspace_bytes(const moe_dims* dims, int32_t n_sample) {
  if (check_dims(dims) != MOE_OK || n_sample < 1 || n_sample > kAuditMaxSamples) return 0;
  return audit_workspace_bytes(n_sample, dims->top_k, dims->D, std::max(dims->I, dims->I_shared));
}

int moe_audit(const moe_dims* dims, const moe_weights* w, const void* x, const int32_t* packed, const void* y,
              const int32_t* sample, int32_t n_sample, float* ref_out, float* result, void* ws, size_t ws_bytes,
              void* stream) {
  int st = check_dims(dims);
  if (st != MOE_OK) return st;
  const moe_dims& d = *dims;
  if (n_sample < 1 || n_sample > kAuditMaxSamples) return MOE_ERR_BAD_DIMS;
  if (d.D > kAuditMaxWidth || d.I > kAuditMaxWidth || d.I_shared > kAuditMaxWidth) return MOE_ERR_UNSUPPORTED;
  if (!w || !x || !packed || !y || !sample || !result || !ws || !w->w_gate || !w->w_up || !w->w_down)
    return MOE_ERR_NULL_ARG;
  if (d.w_dtype == MOE_E4M3 && (!w->s_gate || !w->s_up || !w->s_down)) return MOE_ERR_NULL_ARG;
  if (d.I_shared > 0 && w->sh_gate && (!w->sh_up || !w->sh_down)) return MOE_ERR_NULL_ARG;
  if (d.T == 0) return MOE_ERR_BAD_DIMS;
  if (ws_bytes < audit_workspace_bytes(n_sample, d.top_k, d.D, std::max(d.I, d.I_shared))) return MOE_ERR_WORKSPACE;
  AuditLaunch l{};
  l.x = x; l.packed = packed; l.y = y; l.sample = sample;
  l.T = d.T; l.D = d.D; l.k = d.top_k; l.I = d.I; l.I_shared = d.I_shared; l.e_begin = d.expert_begin;
  l.n_local = d.n_local; l.n_sample = n_sample;
  l.act_el = d.act_dtype == MOE_F32 ? EL_F32 : EL_BF16; l.w_el = w_el(d); l.out_el = d.out_dtype;
  l.packed_layout = d.weight_layout == MOE_LAYOUT_PACKED;
  l.w_gate = w->w_gate; l.w_up = w->w_up; l.w_down = w->w_down;
  l.s_gate = w->s_gate; l.s_up = w->s_up; l.s_down = w->s_down;
  l.sh_gate = d.I_shared > 0 ? w->sh_gate : nullptr; l.sh_up = w->sh_up; l.sh_down = w->sh_down;
  l.ref_out = ref_out; l.result = result; l.ws = ws;
  return hip_status(launch_audit(l, static_cast<hipStream_t>(stream)));
}

int moe_pack_weights(int32_t dtype, int64_t n_mats, int32_t rows, int32_t cols, const void* src, void* dst,
                     void* stream) {
  if (dtype != MOE_F32 && dtype != MOE_BF16 && dtype != MOE_E4M3) return MOE_ERR_UNSUPPORTED;
  if (n_mats < 0 || rows < 0 || cols < 0) return MOE_ERR_BAD_DIMS;
  const int es = dtype == MOE_F32 ? 4 : dtype == MOE_BF16 ? 2 : 1;
  const int64_t row_bytes = static_cast<int64_t>(cols) * es;
  if (rows % 16 || row_bytes % 64 || row_bytes > (1ll << 30)) return MOE_ERR_UNSUPPORTED;
  if (n_mats == 0 || rows == 0 || cols == 0) return MOE_OK;
  if (!src || !dst) return MOE_ERR_NULL_ARG;
  return hip_status(launch_pack(src, dst, n_mats, rows, static_cast<int>(row_bytes),
                                static_cast<hipStream_t>(stream)));
}

int moe_hbm_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (bytes % 16) return MOE_ERR_UNSUPPORTED;
  if (bytes == 0) return MOE_OK;
  if (!buf || !sink) return MOE_ERR_NULL_ARG;
  return hip_status(launch_read_probe(buf, static_cast<int64_t>(bytes), sink, static_cast<hipStream_t>(stream)));
}

int moe_mfma_peak_probe(int32_t dtype, int32_t iters, float* sink, void* stream) {
  if (dtype != MOE_BF16 && dtype != MOE_E4M3) return MOE_ERR_UNSUPPORTED;
  if (iters < 1) return MOE_ERR_BAD_DIMS;
  if (!sink) return MOE_ERR_NULL_ARG;
  return hip_status(launch_mfma_probe(dtype, iters, sink, static_cast<hipStream_t>(stream)));
}

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL_ARG: return "a required pointer argument is NULL";
    case MOE_ERR_BAD_DIMS: return "invalid dimensions";
    case MOE_ERR_UNSUPPORTED: return "unsupported dimensions or dtype combination";
    case MOE_ERR_WORKSPACE: return "workspace smaller than moe_workspace_bytes()";
    case MOE_ERR_HIP: return "HIP kernel launch failed";
    case MOE_ERR_SCRATCH_LIMIT: return "the dims need more scratch than the library's static MOE_STATIC_SCRATCH_BYTES";
    default: return "unknown status";
  }
}

int moe_last_hip_error(void) { return g_last_hip_error; }

int moe_abi_version(void) { return 4; }

}  // extern "C"
