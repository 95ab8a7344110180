// Host-side launch interface of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kMaxLocalExperts = 1024;  // LDS histogram rows of the permutation
constexpr int kPermUnit = 1024;         // (token, slot) pairs per permutation wave

inline int perm_units(int T, int k) { return (T * k + kPermUnit - 1) / kPermUnit; }

// One GEMM problem of the grouped expert kernels.  Rows of group g are
// [offsets[g], offsets[g+1]) (or one group of `rows` rows when offsets is NULL);
// row r of a group reads A row perm[r] (or r when perm is NULL).  Weights are
// [n_groups][N][K] ([out][in]); out is [rows][ldo] at the grouped row index.
struct GemmProblem {
  const void* a;
  const int32_t* perm;
  const float* a_scale;        // E4M3: per A-source-row scale
  int lda;                     // elements
  const int32_t* offsets;      // device, [n_groups + 1], or NULL
  const int32_t* tile_prefix;  // device, [n_groups + 1] M-tile prefix for this kernel's BM
  int n_groups;
  int rows;                    // rows of the single group when offsets is NULL
  const void* w0;              // gate (SwiGLU) or the only weight
  const void* w1;              // up (SwiGLU)
  const float* s0;             // E4M3 per-output-channel scales [n_groups][N]
  const float* s1;
  long long w_stride;          // elements between consecutive groups' weights
  void* out;
  int ldo;                     // elements
  int N, K;
  int k_splits;                // single-group problems only: K is cut into k_splits equal ranges,
  long long out_split_stride;  // each writing its partial product at out + split * out_split_stride
  // Fused unpermute-combine (single-group, non-SwiGLU problems: the shared expert's down
  // projection).  With comb_rows set, out row t is
  //   sum_j w[t][j] * comb_rows[inv[t][j]]  (slot order, inv < 0 skipped)  +  (A W0^T)[t]
  // in fp32, rounded once; comb_rows is [*][ldo] of the output type.
  const void* comb_rows;
  const int32_t* comb_packed;  // [rows][2][comb_k] routing blob (weights from plane 1)
  const int32_t* comb_inv;     // [rows][comb_k] grouped row of each slot, or -1
  int comb_k;
};

// Launch shapes of the grouped GEMM (see gemm.hip):
//   stream16 / stream32: 16- or 32-row M-tiles, 8-step K blocks, non-temporal weight
//                        stream (few rows per expert: decode);
//   tile256:             256-row M-tiles, 2-step K blocks, one workgroup per CU
//                        (many rows per expert: prefill).
enum : int { kShapeStream16 = 0, kShapeStream32 = 1, kShapeTile256 = 2 };

constexpr int gemm_bm(int shape) { return shape == kShapeStream16 ? 16 : shape == kShapeStream32 ? 32 : 256; }
// 16-column output fragments per wave (per matrix for SwiGLU).  el: weight element type;
// packed: fragment-major weights.  Host tile counts and kernels both take it from here.
constexpr int gemm_nf(bool swiglu, int shape, int el, bool packed) {
  return shape == kShapeTile256 ? (swiglu || el == EL_E4M3 || packed ? 2 : 4)
                                : shape == kShapeStream16 ? (swiglu ? 1 : 4) : (swiglu ? 1 : 2);
}
// Output channels per workgroup (4 waves).
constexpr int gemm_bn(bool swiglu, int shape, int el, bool packed) {
  return 4 * gemm_nf(swiglu, shape, el, packed) * 16;
}

// fp32 shadow of the layer on sampled tokens (numerical audit); element types are EL_*.
struct AuditLaunch {
  const void* x;
  const int32_t* packed;
  const void* y;
  const int32_t* sample;
  int T, D, k, I, I_shared, e_begin, n_local, n_sample;
  int act_el, w_el, out_el, packed_layout;
  const void* w_gate;
  const void* w_up;
  const void* w_down;
  const float* s_gate;
  const float* s_up;
  const float* s_down;
  const void* sh_gate;
  const void* sh_up;
  const void* sh_down;
  float* ref_out;
  float* result;
  void* ws;
};
constexpr int kAuditMaxSamples = 4096;
constexpr int kAuditMaxWidth = 16384;  // D and I limits (one fp32 vector in LDS)
size_t audit_workspace_bytes(int n_sample, int k, int D, int i_max);
hipError_t launch_audit(const AuditLaunch& l, hipStream_t stream);

// Fused router projection + top-k (act: bf16 or fp32 codes of EL_*): per (token block,
// expert slice) top-k candidates, then an exact merge per token.  logits_out (nullable)
// receives the fp32 logits.  Scratch: cand_key / cand_id [T][n_slices][k], stats
// [T][n_slices] with n_slices = router_fused_slices(T, E).
constexpr int kFusedSmallT = 2048;          // up to this many tokens: 16-token blocks, 64-expert slices
constexpr int kMaxFusedCandidates = 512;    // slices (E / 64 <= 16) x top_k (<= 32)
int router_fused_slices(int T, int E);
hipError_t launch_router_topk(int el, const void* x, const void* w_router, const float* bias, int T, int D, int E,
                              int k, int renormalize, float* logits_out, int32_t* packed, float* cand_key,
                              int32_t* cand_id, float2* stats, hipStream_t stream);

// Top-k routing.  When n_parts > 1, the logits are the sum of n_parts partial products
// parts[p][T][E] (added in order p = 0, 1, ...), written to `logits` before routing.
hipError_t launch_route(const float* parts, int n_parts, float* logits, const float* bias, int T, int E, int k,
                        int renormalize, int32_t* packed, hipStream_t stream);

// Grouping by expert.  Also writes the M-tile prefixes of both grouped GEMMs (tile heights
// bm0, bm1) into prefix0 / prefix1 ([n_local + 1]), and into *err_word the number of
// pairs whose id lies outside [0, E) (skipped like any non-local pair).
//   hist, base: [perm_units(T, k)][n_local] scratch; rank: [T * k] scratch;
//   bad: [perm_units(T, k)] scratch.
hipError_t launch_permute(const int32_t* packed, int T, int k, int E, int e_begin, int n_local, int32_t* hist,
                          int32_t* base, int32_t* rank, int32_t* bad, int32_t* counts, int32_t* offsets,
                          int32_t* perm_token, int32_t* inv_pos, int bm0, int bm1, int32_t* prefix0,
                          int32_t* prefix1, int32_t* err_word, hipStream_t stream);

hipError_t launch_gather_rows(const void* src, const float* src_scale, const int32_t* perm_token,
                              const int32_t* n_rows_dev, int max_rows, int row_bytes, void* dst, float* dst_scale,
                              hipStream_t stream);

// Per-row E4M3 quantisation.  skip_inv (nullable): inv_pos [rows][skip_k]; rows whose slots are
// all non-local are skipped (left unwritten: the grouped GEMMs never read them).
hipError_t launch_quant_rows(int in_el, const void* src, int rows, const int32_t* n_rows_dev, int cols, void* dst,
                             float* scale, hipStream_t stream, const int32_t* skip_inv = nullptr, int skip_k = 0);

hipError_t launch_tile_prefix(const int32_t* offsets, int n_groups, int bm0, int bm1, int32_t* prefix0,
                              int32_t* prefix1, hipStream_t stream);

// Grouped GEMM of one problem.
//   swiglu: out = silu(A W0^T) * (A W1^T);  else out = A W0^T.
//   el: operand type (EL_F32 / EL_BF16 / EL_E4M3); out_el: EL_F32 / EL_BF16.
//   shape: kShapeStream16 / kShapeStream32 / kShapeTile256.
//   packed: weights in the fragment-major layout of moe_pack_weights (else row-major).
//   max_tiles: host upper bound of the problem's tiles (the grid; surplus workgroups exit).
hipError_t launch_gemm(int el, int out_el, bool swiglu, int shape, bool packed, const GemmProblem& p, int max_tiles,
                       hipStream_t stream);

// The same GEMM with the fused combine epilogue (p.comb_* set; no SwiGLU): el and out_el
// EL_F32 / EL_F32 or EL_BF16 / EL_BF16 or EL_BF16 / EL_F32, shape kShapeStream32 or
// kShapeTile256.
hipError_t launch_gemm_combine(int el, int out_el, int shape, bool packed, const GemmProblem& p, int max_tiles,
                               hipStream_t stream);

// Repack n_mats row-major [rows][row_bytes] matrices into the fragment-major layout.
// Streaming read of bytes (multiple of 16) at src; sink receives one word per workgroup
// (at most kReadProbeBlocks workgroups).
constexpr int kReadProbeBlocks = 16384;
hipError_t launch_read_probe(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream);

// MFMA throughput probe: kMfmaProbeBlocks workgroups of 4 waves, each wave iters x 8 MFMAs
// (bf16 16x16x32 or E4M3 16x16x128); sink receives one float per workgroup.
constexpr int kMfmaProbeBlocks = 2048;
hipError_t launch_mfma_probe(int el, int iters, float* sink, hipStream_t stream);

hipError_t launch_pack(const void* src, void* dst, int64_t n_mats, int rows, int row_bytes, hipStream_t stream);

hipError_t launch_combine(int out_el, const void* out_rows, const int32_t* packed, const int32_t* inv_pos,
                          const void* shared_out, int T, int D, int k, void* y, hipStream_t stream);

}  // namespace moe
