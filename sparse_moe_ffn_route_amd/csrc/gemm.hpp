// Host-side interface of the grouped GEMM kernel (internal to the library): the problem
// description, the launch shapes and the launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace moe {

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
// Waves per workgroup: the tile shape's single-matrix launches with row-major weights (the
// router projection) run 8, two per SIMD; every other launch runs 4.  el: weight element
// type; packed: fragment-major weights.
constexpr int gemm_nw(bool swiglu, int shape, int el, bool packed) {
  return shape == kShapeTile256 && !swiglu && !(el == EL_E4M3 || packed) ? 8 : 4;
}
// 16-column output fragments per wave (per matrix for SwiGLU).  Host tile counts and
// kernels both take it from here.
constexpr int gemm_nf(bool swiglu, int shape, int el, bool packed) {
  return shape == kShapeTile256 ? 2 : shape == kShapeStream16 ? (swiglu ? 1 : 4) : (swiglu ? 1 : 2);
}
// Output channels per workgroup.
constexpr int gemm_bn(bool swiglu, int shape, int el, bool packed) {
  return gemm_nw(swiglu, shape, el, packed) * gemm_nf(swiglu, shape, el, packed) * 16;
}

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

}  // namespace moe
