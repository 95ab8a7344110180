/*
 * moe.h - C ABI of the routed Mixture-of-Experts FFN layer for AMD MI355X (gfx950).
 *
 * The layer (as stated on the pages this library follows):
 *   - hidden size D, E small routed experts of intermediate size I, a router that
 *     keeps the top_k experts of each token through a softmax, and one always-on
 *     shared expert ("Systems Engineering Playbook: Qwen 3.5 MoE on Ironwood TPU",
 *     section "The Architectural Constraints That Break Naive Sharding";
 *     "Tối ưu hóa mô hình Qwen 3.5-397B MoE trên hạ tầng TPU Ironwood", section
 *     "3. Sparse Mixture-of-Experts (MoE)");
 *   - tokens grouped by expert for grouped GEMMs, then unpermuted with a local
 *     reduction (Playbook, table "Three High-Leverage Optimizations");
 *   - under expert parallelism one device owns a contiguous slice of the experts,
 *     receives the routing of all gathered tokens as one packed 32-bit blob of ids
 *     and weights, and returns partial sums for a reduce-scatter (Playbook, section
 *     "Fusing Three Collectives Into Two"; "Como o Google otimizou o Qwen 3.5 de
 *     397B no TPU7x (Ironwood)", section "O problema do sharding e a solução").
 *
 * Readings where the pages are silent: routing = softmax over all E fp32 keys,
 * top_k by (key descending, expert index ascending), weights renormalised over the
 * kept experts; experts are SwiGLU, out = W_down (silu(W_gate x) * W_up x); the
 * shared expert has the same form and is added with weight one.
 *
 * Conventions for every entry point
 *   - All tensor arguments are DEVICE pointers, row-major, owned by the caller,
 *     allocated on the current HIP device.  `dims` and `weights` structs are HOST
 *     pointers read during the call only.
 *   - Weights are stored [out][in] (the reduction dimension is contiguous):
 *       w_router [E][D], w_gate / w_up [n_local][I][D], w_down [n_local][D][I],
 *       shared gate / up [I_shared][D], shared down [D][I_shared].
 *   - The packed routing blob is int32 [T][2][top_k]: plane 0 holds expert ids,
 *     plane 1 the IEEE binary32 bits of the matching weights (token-major, so the
 *     blobs of several devices concatenate along tokens).
 *   - Every call is asynchronous on `stream` (a hipStream_t passed as void*; NULL
 *     is the default stream).  The library never allocates, frees or synchronises;
 *     scratch memory is the caller's `ws` buffer of at least moe_workspace_bytes(dims)
 *     bytes, which must not be shared by calls that may run concurrently.  The one
 *     piece of global state is the static device scratch of moe_layer_forward_noalloc
 *     (and the per-device table of its addresses).
 *   - Arguments are validated on the host before any launch; on error nothing is
 *     launched and a negative moe_status is returned.  T = 0 is a successful no-op.
 *   - Results are deterministic: ids, counts, offsets, permutation are unique
 *     integers, and every floating-point sum has a fixed order.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage types. */
enum moe_dtype {
  MOE_F32 = 0,  /* IEEE binary32 */
  MOE_BF16 = 1, /* bfloat16 */
  MOE_E4M3 = 2  /* OCP FP8 E4M3 (max 448, no infinities), weights only, with fp32 scales */
};

/* Return codes. */
enum moe_status {
  MOE_OK = 0,
  MOE_ERR_NULL_ARG = -1,    /* a required pointer is NULL */
  MOE_ERR_BAD_DIMS = -2,    /* T < 0, D/E/I/top_k < 1, top_k > E, expert slice outside [0, E) */
  MOE_ERR_UNSUPPORTED = -3, /* dtype combination, D or I not a multiple of 64, E > 1024, top_k > 32,
                               one expert's or the router's weight matrix of 2 GiB or more */
  MOE_ERR_WORKSPACE = -4,   /* ws_bytes smaller than moe_workspace_bytes(dims) */
  MOE_ERR_HIP = -5,         /* a kernel launch failed (see moe_last_hip_error) */
  MOE_ERR_SCRATCH_LIMIT = -6 /* moe_layer_forward_noalloc: the dims need more than MOE_STATIC_SCRATCH_BYTES */
};

/*
 * Error word of a workspace: the int32 at byte offset MOE_WS_ERROR_OFFSET of `ws` holds,
 * after a moe_permute or moe_layer_forward call on that workspace has run, the number of
 * (token, slot) pairs of the routing blob whose expert id lies outside [0, E).  Such a
 * pair is skipped like a pair of another device's expert; a non-zero count means the
 * blob was corrupt (the blob may arrive from another device: Playbook, section "Fusing
 * Three Collectives Into Two").  The word is rewritten by every such call (never
 * accumulated), so it needs no clearing; read it after the call has completed on its
 * stream.
 */
#define MOE_WS_ERROR_OFFSET 0

/* Problem shape. */
typedef struct moe_dims {
  int32_t T;            /* tokens (rows of x) */
  int32_t D;            /* hidden size */
  int32_t E;            /* routed experts of the whole layer */
  int32_t top_k;        /* experts kept per token */
  int32_t I;            /* intermediate size of a routed expert */
  int32_t I_shared;     /* intermediate size of the shared expert; 0 = no shared expert */
  int32_t expert_begin; /* first local expert id (0 for the whole layer) */
  int32_t n_local;      /* local experts: ids expert_begin .. expert_begin + n_local - 1 */
  int32_t renormalize;  /* 1: kept weights sum to 1; 0: kept softmax entries as they are */
  int32_t act_dtype;    /* x, router weight, shared weights: MOE_F32 or MOE_BF16 */
  int32_t w_dtype;      /* routed expert weights: MOE_F32 (with act F32), MOE_BF16 or MOE_E4M3 (with act BF16) */
  int32_t out_dtype;    /* y and expert outputs: MOE_F32 or MOE_BF16 */
  int32_t weight_layout;/* routed and shared expert weights: MOE_LAYOUT_ROWS or MOE_LAYOUT_PACKED */
} moe_dims;

/* Storage order of the expert weight matrices (router weights are always MOE_LAYOUT_ROWS). */
enum moe_layout {
  MOE_LAYOUT_ROWS = 0,   /* row-major [out][in] */
  MOE_LAYOUT_PACKED = 1  /* fragment-major, as written by moe_pack_weights */
};

/* Weights of the layer (device pointers). */
typedef struct moe_weights {
  const void* w_router;  /* [E][D] act_dtype; may be NULL when routing is given */
  const void* w_gate;    /* [n_local][I][D] w_dtype */
  const void* w_up;      /* [n_local][I][D] w_dtype */
  const void* w_down;    /* [n_local][D][I] w_dtype */
  const float* s_gate;   /* [n_local][I] per-output-channel scales (E4M3 only, else NULL) */
  const float* s_up;     /* [n_local][I] */
  const float* s_down;   /* [n_local][D] */
  const void* sh_gate;   /* [I_shared][D] act_dtype (NULL if I_shared == 0) */
  const void* sh_up;     /* [I_shared][D] */
  const void* sh_down;   /* [D][I_shared] */
} moe_weights;

/*
 * Scratch bytes needed by any entry point for these dims (upper bound over all
 * routings).  Returns 0 if the dims are invalid.
 */
size_t moe_workspace_bytes(const moe_dims* dims);

/*
 * Router: top-k selection and weights, written as the packed blob.
 *   logits[t][e] = sum_d x[t][d] * w_router[e][d]   (fp32 accumulation)
 *   key = fp32(logit + logit_bias[e]); keep the top_k keys (larger first, equal
 *   key -> lower expert id); w_j = exp(key_j - key_0) / sum_i exp(key_i - key_0)
 *   over the kept keys (renormalize = 1), or over all E (renormalize = 0).
 * Source: the router of "3. Sparse Mixture-of-Experts (MoE)" (Tối ưu hóa ... TPU
 * Ironwood); the packed blob of Playbook "Fusing Three Collectives Into Two".
 *
 *   x          [T][D] act_dtype, or NULL
 *   w_router   [E][D] act_dtype, or NULL
 *   logits     [T][E] fp32: OUTPUT when x and w_router are given; INPUT when both
 *              are NULL (route from caller-supplied logits).
 *   logit_bias [E] fp32 or NULL (an additive popularity bias; -inf never chosen).
 *              Each token needs at least top_k finite keys; NaN is not supported.
 *   packed     [T][2][top_k] int32 output.
 *   ws         scratch of ws_bytes >= moe_workspace_bytes(dims), or NULL.  With scratch, a
 *              small-T projection is split along D into partial products that the
 *              routing kernel adds in a fixed order (same result on every call).
 */
int moe_route(const moe_dims* dims, const void* x, const void* w_router, float* logits,
              const float* logit_bias, int32_t* packed, void* ws, size_t ws_bytes, void* stream);

/*
 * The same routing as moe_route with x and w_router given, with the top-k selection
 * fused into the kernel that produces the logits (the open item of Playbook "The
 * Remaining Roadmap"): each workgroup computes the logits of a block of tokens against a
 * slice of 64 (or, above 2048 tokens, 128) experts with MFMAs in fp32 and keeps each
 * token's top_k of that slice as candidates (key, id); a second kernel merges every
 * token's candidates of all slices into its top_k with the same order, which is exact
 * because the global top_k lies in the union of the slices' top_k.  The fp32 logits never
 * go to memory unless `logits` asks for a copy.
 *
 *   x, w_router, logit_bias, packed   as for moe_route (x and w_router required)
 *   logits     [T][E] fp32 output copy of the logits, or NULL for none
 *   ws         scratch of ws_bytes >= moe_workspace_bytes(dims) (the candidates)
 * Needs x and w_router each below 2 GiB, else MOE_ERR_UNSUPPORTED.  The ids and weights
 * equal moe_route's for the same fp32 logits; the logits themselves may differ by
 * summation order (both within the fp32 accumulation bound).
 */
int moe_route_fused(const moe_dims* dims, const void* x, const void* w_router, float* logits,
                    const float* logit_bias, int32_t* packed, void* ws, size_t ws_bytes, void* stream);

/*
 * Permutation: group the (token, slot) pairs whose expert is local by expert
 * (experts ascending, (t, j) ascending inside an expert), the grouping that the
 * grouped GEMMs and the later "unpermutation + local reduction" need (Playbook,
 * introduction and table "Three High-Leverage Optimizations"); under expert
 * parallelism only the device's own slice of experts is grouped (Playbook, section
 * "Fusing Three Collectives Into Two").  Ids outside the local slice (other devices'
 * experts) are skipped; ids outside [0, E) are skipped too and counted in the error
 * word at ws + MOE_WS_ERROR_OFFSET.
 *
 *   packed     [T][2][top_k] int32 input
 *   counts     [n_local] int32 out: rows of each local expert
 *   offsets    [n_local + 1] int32 out: exclusive prefix sum; offsets[n_local] = N_a
 *   perm_token [T * top_k] int32 out: first N_a entries = source token of each row
 *   inv_pos    [T][top_k] int32 out: grouped row of (t, j), or -1 if not local
 *   x          [T][D] act_dtype, optional (NULL: index-only)
 *   x_perm     [T * top_k][D] optional gather target: act_dtype, or E4M3 codes when
 *              w_dtype is E4M3 (x is then quantised per token first)
 *   x_perm_scale [T * top_k] fp32, E4M3 only: per-row dequantisation scale
 */
int moe_permute(const moe_dims* dims, const int32_t* packed, int32_t* counts, int32_t* offsets,
                int32_t* perm_token, int32_t* inv_pos, const void* x, void* x_perm,
                float* x_perm_scale, void* ws, size_t ws_bytes, void* stream);

/*
 * Grouped SwiGLU experts on ragged groups:
 *   for each local expert e and each row r in [offsets[e], offsets[e+1]):
 *     h = silu(W_gate[e] a_r) * (W_up[e] a_r);  out_rows[r] = W_down[e] h
 * Source: the "Grouped GEMMs" block of the Playbook's introduction and table.
 *
 *   a_rows     if perm_token is NULL: grouped rows [N_a][D]; else x [T][D] and row r
 *              reads x[perm_token[r]].  act_dtype, or E4M3 codes when w_dtype is E4M3.
 *   a_scale    E4M3 only: fp32 scale per row of a_rows ([N_a], or [T] with perm_token)
 *   perm_token [N_a] int32 or NULL
 *   offsets    [n_local + 1] int32 (device)
 *   weights    local slice, see moe_weights; scales only for E4M3
 *   out_rows   [T * top_k][D] out_dtype: unweighted expert outputs of the grouped rows
 * The shared expert is not part of this call (call it with n_local = 1,
 * offsets = {0, T}, perm_token = NULL and I = I_shared to evaluate it alone).
 */
int moe_grouped_ffn(const moe_dims* dims, const void* a_rows, const float* a_scale,
                    const int32_t* perm_token, const int32_t* offsets, const void* w_gate,
                    const void* w_up, const void* w_down, const float* s_gate, const float* s_up,
                    const float* s_down, void* out_rows, void* ws, size_t ws_bytes, void* stream);

/*
 * Unpermute and reduce ("unpermutation + local reduction", Playbook table
 * "Three High-Leverage Optimizations"):
 *   y[t] = sum_{j : inv_pos[t][j] >= 0} w[t][j] * out_rows[inv_pos[t][j]]  (+ shared_out[t])
 * summed in fp32 in slot order, the shared row added last, rounded once to out_dtype.
 *
 *   out_rows   [N_a][D] out_dtype
 *   packed     [T][2][top_k] int32 (weights are read from plane 1)
 *   inv_pos    [T][top_k] int32
 *   shared_out [T][D] out_dtype or NULL
 *   y          [T][D] out_dtype
 */
int moe_unpermute_combine(const moe_dims* dims, const void* out_rows, const int32_t* packed,
                          const int32_t* inv_pos, const void* shared_out, void* y, void* stream);

/*
 * The whole layer: route -> permute -> grouped experts (+ shared expert) -> combine.
 * The layer of "3. Sparse Mixture-of-Experts (MoE)" (Tối ưu hóa ... TPU Ironwood):
 * top-k routed experts plus the always-on shared expert; its dataflow of grouped GEMMs
 * followed by unpermutation with a local reduction is the Playbook's (introduction and
 * table "Three High-Leverage Optimizations"); with a local slice and given routing it is
 * one device's expert-parallel share between the all-gather and the reduce-scatter
 * (Playbook, "Fusing Three Collectives Into Two"; "Como o Google otimizou ...",
 * section "O problema do sharding e a solução").  A given blob's ids outside [0, E)
 * are counted in the error word at ws + MOE_WS_ERROR_OFFSET.
 *
 *   x          [T][D] act_dtype
 *   packed_in  [T][2][top_k] int32 or NULL.  Non-NULL: the routing is given (one
 *              device's expert-parallel share) and the router is skipped.
 *   logit_bias [E] fp32 or NULL (router only)
 *   y          [T][D] out_dtype.  With a local slice: the slice's partial sums
 *              (zero rows for tokens without a local expert).
 *   logits_out [T][E] fp32 or NULL: copy of the router logits
 *   packed_out [T][2][top_k] int32 or NULL: copy of the routing blob
 *   stage_events NULL, or MOE_STAGE_EVENTS caller-created hipEvent_t handles (as
 *              void*) that are recorded on `stream` at the stage boundaries: [0] before
 *              routing, [1] after routing, [2] after grouping (and the fp8 quantisation
 *              of x), [3] after the routed gate/up GEMM, [4] after the routed down GEMM
 *              (and the fp8 quantisation of h), [5] after the shared expert's two GEMMs,
 *              [6] after the combine.  With a shared expert the combine runs inside the
 *              shared expert's down projection, so [5] and [6] mark the same point.  Only
 *              for timing; the kernels are the same either way.
 * With a shared expert, y[t] = (sum over the slots in order of w * expert row, in fp32)
 * + the shared expert's fp32 output, rounded once; without one, the slot sum alone.
 */
#define MOE_STAGE_EVENTS 7
int moe_layer_forward(const moe_dims* dims, const moe_weights* weights, const void* x,
                      const int32_t* packed_in, const float* logit_bias, void* y, float* logits_out,
                      int32_t* packed_out, void* ws, size_t ws_bytes, void* const* stage_events,
                      void* stream);

/*
 * moe_layer_forward for callers that cannot allocate device memory or pass a workspace
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Scratch is a static device array of MOE_STATIC_SCRATCH_BYTES inside the library: each
 * GPU the library runs on holds its own copy until the process ends.  The array's
 * address on the current device is looked up once per device on the first call; the
 * call itself allocates nothing and launches the same kernels as moe_layer_forward, so
 * its results are the same bit for bit.
 *
 *   arguments  as for moe_layer_forward, without ws / ws_bytes
 *   bad_ids    device int32 or NULL: receives the error word (ids outside [0, E) in the
 *              routing blob), since the static scratch is not visible to the caller
 * Returns MOE_ERR_SCRATCH_LIMIT (nothing launched) when moe_workspace_bytes(dims)
 * exceeds MOE_STATIC_SCRATCH_BYTES; the 512-token decode batch of the D = 4096,
 * E = 512, I = 1024 layer fits, 8192-token prefill batches do not.
 * Every call on one GPU shares that GPU's array and leaves its contents behind: calls
 * that may overlap on one GPU (several streams, several host threads) race and must
 * be serialised by the caller.  Nothing in the array needs to start at zero.
 */
#define MOE_STATIC_SCRATCH_BYTES (96u << 20)
int moe_layer_forward_noalloc(const moe_dims* dims, const moe_weights* weights, const void* x,
                              const int32_t* packed_in, const float* logit_bias, void* y, float* logits_out,
                              int32_t* packed_out, int32_t* bad_ids, void* const* stage_events, void* stream);

/*
 * Repack weight matrices from row-major [out][in] into the fragment-major order the
 * grouped GEMM streams: for each block of 16 output rows ("fragment") and each 64-byte
 * slice of the reduction dimension, the 16 x 64 bytes are stored as one contiguous
 * 1 KB run, lane l of the run holding 16 bytes of row (l % 16) at byte (l / 16) * 16 of
 * the slice.  Every load instruction of the GEMM then reads whole contiguous 1 KB runs
 * and every fragment is read front to back.  This is a one-time transform at weight
 * load time; the values are not changed.
 *
 *   dtype   MOE_F32, MOE_BF16 or MOE_E4M3 (element size of src / dst)
 *   n_mats  number of [rows][cols] matrices stored back to back (e.g. n_local experts)
 *   rows    output rows per matrix (multiple of 16)
 *   cols    reduction length per row; cols * element size must be a multiple of 64
 *   src     device, n_mats * rows * cols elements, row-major
 *   dst     device, same size, must not overlap src
 * Pack w_gate / w_up as (n_local, I, D), w_down as (n_local, D, I), the shared expert's
 * gate / up as (1, I_shared, D) and its down as (1, D, I_shared), then set
 * dims.weight_layout = MOE_LAYOUT_PACKED.  Returns MOE_ERR_BAD_DIMS / MOE_ERR_UNSUPPORTED
 * for sizes outside these rules, MOE_ERR_NULL_ARG for NULL pointers.
 */
int moe_pack_weights(int32_t dtype, int64_t n_mats, int32_t rows, int32_t cols, const void* src, void* dst,
                     void* stream);

/*
 * Numerical audit: an fp32 shadow of the layer on sampled tokens, compared with the
 * layer's output.  For each sampled token t the reference is
 *   ref[t] = sum_j w[t][j] * W_down (silu(W_gate x_t) * (W_up x_t)) over the local slots
 *            of `packed`, in slot order, + the shared expert (weight 1) if present,
 * evaluated in fp32 from the stored tensors: E4M3 weights decoded and scaled per channel,
 * x and h never quantised, SwiGLU with an IEEE division.  It measures what the fast
 * path's bf16 rounding and fp8 quantisation cost, as the "Numerical Verification Layer"
 * of Playbook "Roofline Validation" checks low-precision results against a
 * high-precision evaluation.
 *
 *   dims, weights  as for moe_layer_forward (same layout, local slice and dtypes)
 *   x         [T][D] act_dtype: the hidden states the layer was run on
 *   packed    [T][2][top_k] int32: the routing the layer used (e.g. its packed_out)
 *   y         [T][D] out_dtype: the layer's output to audit
 *   sample    [n_sample] int32 device token indices in [0, T) (clamped into range)
 *   n_sample  1 .. 4096
 *   ref_out   [n_sample][D] fp32 output copy of the reference rows, or NULL
 *   result    [2] fp32 device output: max |y - ref| and max |ref| over the samples
 *   ws        scratch of ws_bytes >= moe_audit_workspace_bytes(dims, n_sample)
 * Limits: D, I, I_shared <= 16384 (MOE_ERR_UNSUPPORTED).  T = 0 is MOE_ERR_BAD_DIMS
 * (nothing to sample).  Not a hot path: it reads every sampled token's expert weights
 * once per token.
 */
size_t moe_audit_workspace_bytes(const moe_dims* dims, int32_t n_sample);
int moe_audit(const moe_dims* dims, const moe_weights* weights, const void* x, const int32_t* packed,
              const void* y, const int32_t* sample, int32_t n_sample, float* ref_out, float* result, void* ws,
              size_t ws_bytes, void* stream);

/*
 * Measurement helper, not part of the layer: reads `bytes` (a multiple of 16) of device
 * memory at buf once with wide non-temporal loads and writes 16384 uint32 words of XOR
 * checksums into sink (device, caller-owned, at least 16384 words).  Timing it over a
 * buffer much larger than the caches gives the achievable HBM read bandwidth that the
 * grouped GEMMs' weight streams are compared with.  Asynchronous on stream.  Returns
 * MOE_ERR_UNSUPPORTED if bytes is not a multiple of 16, MOE_ERR_NULL_ARG for NULL
 * pointers (bytes > 0).
 */
int moe_hbm_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream);

/*
 * Measurement helper, not part of the layer: the matrix cores' sustained rate.  Launches
 * MOE_MFMA_PROBE_BLOCKS workgroups of 4 waves; each wave runs iters rounds of 8
 * independent MFMA accumulator chains on register operands (no memory traffic in the
 * loop): dtype MOE_BF16 issues 16x16x32 bf16 MFMAs (16384 FLOP each), MOE_E4M3 16x16x128
 * E4M3 MFMAs (65536 FLOP each).  FLOP per launch = MOE_MFMA_PROBE_BLOCKS * 4 * 8 * iters *
 * (FLOP per MFMA); timing a launch of a few milliseconds gives the dense MFMA rate at the
 * clock the chip holds under that load, which the grouped GEMMs are compared with.  sink:
 * device, at least MOE_MFMA_PROBE_BLOCKS floats (one sum per workgroup).  Asynchronous on
 * stream.  MOE_ERR_UNSUPPORTED for another dtype, MOE_ERR_BAD_DIMS for iters < 1.
 */
#define MOE_MFMA_PROBE_BLOCKS 2048
int moe_mfma_peak_probe(int32_t dtype, int32_t iters, float* sink, void* stream);

/* Human-readable text of a moe_status code (static storage). */
const char* moe_status_string(int status);

/* hipError_t of the last failed launch on the calling host thread (0 if none). */
int moe_last_hip_error(void);

/* ABI version of this header: 4 (3: MOE_STAGE_EVENTS became 7, with a mark after the shared
 * expert; moe_audit and moe_audit_workspace_bytes were added; 4: the workspace error word,
 * moe_layer_forward_noalloc and moe_mfma_peak_probe). */
int moe_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
