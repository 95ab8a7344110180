// Host-side launch interface of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm.hpp"

namespace moe {

constexpr int kMaxLocalExperts = 1024;  // LDS histogram rows of the permutation
constexpr int kPermUnit = 1024;         // (token, slot) pairs per permutation wave

inline int perm_units(int T, int k) { return (T * k + kPermUnit - 1) / kPermUnit; }

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
// xq_src (nullable): bf16 token rows [T][xq_cols], quantised per row to E4M3 into xq_dst
// [T][xq_cols] and xq_scale [T] as launch_quant_rows does.  On the multi-workgroup path
// every row is quantised by workgroups of the ranking launch, beside the ranking; on the
// one-workgroup path rows without a local slot are skipped (left unwritten) by a launch
// after the grouping.  The grouped GEMMs read only rows with a local slot.
hipError_t launch_permute(const int32_t* packed, int T, int k, int E, int e_begin, int n_local, int32_t* hist,
                          int32_t* base, int32_t* rank, int32_t* bad, int32_t* counts, int32_t* offsets,
                          int32_t* perm_token, int32_t* inv_pos, int bm0, int bm1, int32_t* prefix0,
                          int32_t* prefix1, int32_t* err_word, hipStream_t stream, const void* xq_src = nullptr,
                          int xq_cols = 0, void* xq_dst = nullptr, float* xq_scale = nullptr);

hipError_t launch_gather_rows(const void* src, const float* src_scale, const int32_t* perm_token,
                              const int32_t* n_rows_dev, int max_rows, int row_bytes, void* dst, float* dst_scale,
                              hipStream_t stream);

// Per-row E4M3 quantisation.  skip_inv (nullable): inv_pos [rows][skip_k]; rows whose slots are
// all non-local are skipped (left unwritten: the grouped GEMMs never read them).
hipError_t launch_quant_rows(int in_el, const void* src, int rows, const int32_t* n_rows_dev, int cols, void* dst,
                             float* scale, hipStream_t stream, const int32_t* skip_inv = nullptr, int skip_k = 0);

hipError_t launch_tile_prefix(const int32_t* offsets, int n_groups, int bm0, int bm1, int32_t* prefix0,
                              int32_t* prefix1, hipStream_t stream);



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
