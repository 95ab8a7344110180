// Fused router: projection and top-k selection per (token block, expert slice), then an
// exact merge of the slices' candidates, so the [T][E] fp32 logits never have to go
// through HBM.
//
// Source: the router of "Tối ưu hóa mô hình Qwen 3.5-397B MoE trên hạ tầng TPU Ironwood",
// section "3. Sparse Mixture-of-Experts (MoE)" (projection to the experts, softmax
// distribution, top 10 of 512); fusing the selection into the kernel that produces the
// logits is the open item of "Systems Engineering Playbook: Qwen 3.5 MoE on Ironwood
// TPU", section "The Remaining Roadmap"; routing needs full-precision accumulation
// (Playbook, "Roofline Validation").
//
// Stage 1 (router_slice_kernel): one 256-thread workgroup per (block of TB tokens, slice
// of SW = 64 NFW experts).  Wave w computes the logits of experts w NFW 16 .. + NFW 16 of
// the slice for the TB tokens with 16x16 MFMAs (fp32 accumulation over all of D, in K
// order): W_r rows stream from L2 into registers as the A operand, the token rows are
// staged in LDS per K block as the B operand.  The TB x SW tile goes to LDS; each wave then
// takes its tokens' top-k of the slice by k rounds of a wave arg-best with the order
// "larger key first, then lower expert id" (key = fp32(logit + bias)), and writes them as
// candidates, with the slice's largest key m and sum of exp(key - m) for the
// non-renormalised softmax.  The slice index varies fastest over the grid, so on the 8
// XCDs of an MI355X each XCD serves one slice's W_r from its L2.
// Stage 2 (router_merge_kernel): one wave per token takes the top k of the candidates of
// all slices with the same order.  The global top-k lies in the union of the slices'
// top-k (every expert ahead of a global top-k member in its slice is ahead of it
// globally too), so the selection is exactly the unfused one; the weights are computed
// like select_topk's, from the same kept keys.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "kernels.hpp"
#include "topk.hpp"

namespace moe {

namespace {

constexpr int kWRing = 3;                // weight blocks in the register ring (2 in flight)

// KS: 64-byte K steps per block.  A wave streams the W_r rows of its NFW 16 experts, so its
// bytes in flight are 2 blocks x NFW x KS KB: long blocks keep the stream from being
// latency-bound.  KG: groups of 4 waves that split D into KG equal ranges (a workgroup of
// 256 KG threads); their partial tiles are added in group order in LDS, so the logits
// still have one fixed summation order.
template <int EL, int TB, int NFW, int KS, int KG>
__global__ __launch_bounds__(256 * KG) void router_slice_kernel(const void* __restrict__ x,
                                                                const void* __restrict__ w_router,
                                                                const float* __restrict__ bias, int T, int D, int E,
                                                                int k, int n_slices, float* __restrict__ logits_out,
                                                                float* __restrict__ cand_key,
                                                                int32_t* __restrict__ cand_id,
                                                                float2* __restrict__ stats) {
  constexpr int kKSteps = KS;
  constexpr int kKBlk = kKSteps * 64;     // bytes of each row per K block
  constexpr int kRow = kKBlk + 16;        // padded LDS row of the token tile (bytes)
  constexpr int SW = 4 * NFW * 16;        // experts per slice
  constexpr int MF = TB / 16;             // 16-token B fragments
  constexpr int LOG_ROW = SW + 4;         // padded LDS row of the logits tile (floats)
  constexpr int TOK_BYTES = KG * 2 * TB * kRow;
  constexpr int LOG_BYTES = KG * TB * LOG_ROW * 4;
  constexpr int LDS_BYTES = TOK_BYTES > LOG_BYTES ? TOK_BYTES : LOG_BYTES;
  constexpr int ES = ElSize<EL>::v;
  constexpr int PL = SW / kWave;          // slice keys per lane
  constexpr int NW = 4 * KG;              // waves of the workgroup
  __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];

  const int s = blockIdx.x % n_slices;
  const int t0 = (blockIdx.x / n_slices) * TB;
  const int e0 = s * SW;
  const int gw = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave of the workgroup
  const int kg = gw / 4, wv = gw % 4;                                 // K group, wave in the group
  const int tid = threadIdx.x % 256;                                  // thread in the group
  const int lane = threadIdx.x % kWave, lrow = lane & 15, lgrp = lane >> 4;
  const uint32_t row_bytes = static_cast<uint32_t>(D) * ES;
  // the host keeps row_bytes a multiple of KG * kKBlk
  const int nblk = static_cast<int>(row_bytes / kKBlk) / KG;  // K blocks of this group
  const uint32_t kofs = static_cast<uint32_t>(kg * nblk) * kKBlk;
  uint8_t* tok = lds + kg * 2 * TB * kRow;

  // operand offsets: W_r rows past E and token rows past T re-read the last valid row
  // (their results are never used)
  const __amdgpu_buffer_rsrc_t wres = buffer_rsrc(w_router);
  const __amdgpu_buffer_rsrc_t xres = buffer_rsrc(x);
  uint32_t woff[NFW];
#pragma unroll
  for (int nf = 0; nf < NFW; ++nf) {
    const int e = min(e0 + wv * NFW * 16 + nf * 16 + lrow, E - 1);
    woff[nf] = static_cast<uint32_t>(e) * row_bytes + lgrp * 16;
  }
  constexpr int kCpr = kKBlk / 16;                      // 16-byte chunks per token row per block
  constexpr int kChunks = TB * kCpr;                    // chunks of the token tile per block
  constexpr int kPasses = (kChunks + 255) / 256;
  const int crow = tid / kCpr, ccol = (tid % kCpr) * 16;
  uint32_t toff[kPasses];
#pragma unroll
  for (int i = 0; i < kPasses; ++i) {
    const int t = min(t0 + min(crow + i * (256 / kCpr), TB - 1), T - 1);
    toff[i] = static_cast<uint32_t>(t) * row_bytes + ccol;
  }
  const bool loads_tokens = kChunks >= 256 || tid < kChunks;

  f32x4 acc[NFW][MF];
#pragma unroll
  for (int nf = 0; nf < NFW; ++nf)
#pragma unroll
    for (int mf = 0; mf < MF; ++mf) acc[nf][mf] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 wr[kWRing][NFW][kKSteps];
  u32x4 tv[kPasses];
  auto ld_w = [&](u32x4 (&w)[NFW][kKSteps], int kb) {
    const uint32_t o = kofs + static_cast<uint32_t>(min(kb, nblk - 1)) * kKBlk;
#pragma unroll
    for (int st = 0; st < kKSteps; ++st)
#pragma unroll
      for (int nf = 0; nf < NFW; ++nf) w[nf][st] = buffer_load16(wres, woff[nf], o + st * 64);
  };
  auto ld_t = [&](int kb) {
    const uint32_t o = kofs + static_cast<uint32_t>(min(kb, nblk - 1)) * kKBlk;
#pragma unroll
    for (int i = 0; i < kPasses; ++i) tv[i] = buffer_load16(xres, toff[i], o);
  };
  auto st_t = [&](int buf) {
    if (!loads_tokens) return;
#pragma unroll
    for (int i = 0; i < kPasses; ++i)
      *reinterpret_cast<u32x4*>(&tok[buf * TB * kRow + (crow + i * (256 / kCpr)) * kRow + ccol]) = tv[i];
  };
  auto mm = [&](const u32x4 (&w)[NFW][kKSteps], int buf) {
    const uint8_t* sb = &tok[buf * TB * kRow + lrow * kRow + lgrp * 16];
#pragma unroll
    for (int st = 0; st < kKSteps; ++st)
#pragma unroll
      for (int mf = 0; mf < MF; ++mf) {
        const u32x4 b = *reinterpret_cast<const u32x4*>(sb + mf * 16 * kRow + st * 64);
#pragma unroll
        for (int nf = 0; nf < NFW; ++nf) acc[nf][mf] = mfma_chunk<EL>(w[nf][st], b, acc[nf][mf]);
      }
  };

  // K blocks: weights two blocks ahead in a three-block register ring, token rows one
  // block ahead through registers into the other LDS buffer of the group
  ld_t(0);
  ld_w(wr[0], 0);
  ld_w(wr[1], 1);
  st_t(0);
  __syncthreads();
  for (int kb = 0; kb < nblk; kb += kWRing) {
#pragma unroll
    for (int j = 0; j < kWRing; ++j) {
      if (j > 0 && kb + j >= nblk) break;
      ld_t(kb + j + 1);
      ld_w(wr[(j + 2) % kWRing], kb + j + 2);
      mm(wr[j], (kb + j) & 1);
      st_t((kb + j + 1) & 1);
      __syncthreads();
    }
  }

  // partial logits tiles to LDS (group kg's at kg * TB rows): lane holds experts
  // 4 (l / 16) + r of each fragment for token l % 16; then the groups' partials are added
  // in group order into group 0's tile
  float* lt = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int nf = 0; nf < NFW; ++nf)
#pragma unroll
    for (int mf = 0; mf < MF; ++mf) {
      const int c = wv * NFW * 16 + nf * 16 + lgrp * 4;
      *reinterpret_cast<f32x4*>(&lt[(kg * TB + mf * 16 + lrow) * LOG_ROW + c]) = acc[nf][mf];
    }
  __syncthreads();
  if constexpr (KG > 1) {
    for (int i = threadIdx.x; i < TB * SW; i += 256 * KG) {
      const int r = i / SW, c = i % SW;
      float v = lt[r * LOG_ROW + c];
#pragma unroll
      for (int g = 1; g < KG; ++g) v += lt[(g * TB + r) * LOG_ROW + c];
      lt[r * LOG_ROW + c] = v;
    }
    __syncthreads();
  }

  // each wave: top-k of the slice for its tokens
  for (int r = gw; r < TB; r += NW) {
    const int t = t0 + r;
    if (t >= T) break;
    float key[PL];
    uint32_t taken = 0;  // bit i: slice expert lane + 64 i selected or past E
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const int e = e0 + lane + i * kWave;
      key[i] = -INFINITY;
      if (e < E) {
        const float v = lt[r * LOG_ROW + lane + i * kWave];
        if (logits_out) logits_out[static_cast<size_t>(t) * E + e] = v;
        key[i] = bias ? v + bias[e] : v;  // one fp32 add
      } else {
        taken |= 1u << i;
      }
    }
    // slice statistics for the full-softmax denominator
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < PL; ++i)
      if (!((taken >> i) & 1u)) m = fmaxf(m, key[i]);
    m = wave_max(m);
    float z = 0.0f;
    if (m != -INFINITY) {
#pragma unroll
      for (int i = 0; i < PL; ++i)
        if (!((taken >> i) & 1u)) z += expf(key[i] - m);
    }
    z = wave_sum(z);
    const size_t ts = static_cast<size_t>(t) * n_slices + s;
    if (lane == 0) stats[ts] = make_float2(m, z);
    // k rounds of arg-best; slots of a slice with fewer than k experts get (-inf, E)
    for (int j = 0; j < k; ++j) {
      float bk = -INFINITY;
      int bi = 0x7FFFFFFF;
#pragma unroll
      for (int i = 0; i < PL; ++i) {
        const int e = e0 + lane + i * kWave;
        if (!((taken >> i) & 1u) && key_before(key[i], e, bk, bi)) {
          bk = key[i];
          bi = e;
        }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float ok = __shfl_xor(bk, o, kWave);
        const int oi = __shfl_xor(bi, o, kWave);
        if (key_before(ok, oi, bk, bi)) {
          bk = ok;
          bi = oi;
        }
      }
      if (bi < E && ((bi - e0) & (kWave - 1)) == lane) taken |= 1u << ((bi - e0) / kWave);
      if (lane == 0) {
        cand_key[ts * k + j] = bk;
        cand_id[ts * k + j] = bi < E ? bi : E;
      }
    }
  }
}

// Stage 2: one wave per token; lane l holds candidates l, l + 64, ... of the token's
// n_slices * k candidates.
__global__ __launch_bounds__(256) void router_merge_kernel(const float* __restrict__ cand_key,
                                                           const int32_t* __restrict__ cand_id,
                                                           const float2* __restrict__ stats, int T, int E, int k,
                                                           int n_slices, int renormalize,
                                                           int32_t* __restrict__ packed) {
  constexpr int PL = kMaxFusedCandidates / kWave;
  const int lane = lane_id();
  const int t = blockIdx.x * 4 + threadIdx.x / kWave;
  if (t >= T) return;
  const int nc = n_slices * k;
  const float* ck = cand_key + static_cast<size_t>(t) * nc;
  const int32_t* ci = cand_id + static_cast<size_t>(t) * nc;
  float key[PL];
  int id[PL];
  uint32_t taken = 0;  // bit i: candidate lane + 64 i selected or not an expert
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    const int c = lane + i * kWave;
    key[i] = -INFINITY;
    id[i] = 0x7FFFFFFF;
    if (c < nc) {
      key[i] = ck[c];
      id[i] = ci[c];
    }
    if (c >= nc || id[i] >= E) taken |= 1u << i;
  }
  float sel_key = 0.0f;
  int sel_idx = 0;
  for (int j = 0; j < k; ++j) {
    float bk = -INFINITY;
    int bi = 0x7FFFFFFF, bs = -1;  // bs: candidate slot lane + 64 i of the lane's best
#pragma unroll
    for (int i = 0; i < PL; ++i)
      if (!((taken >> i) & 1u) && key_before(key[i], id[i], bk, bi)) {
        bk = key[i];
        bi = id[i];
        bs = i;
      }
    float wk = bk;
    int wi = bi;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ok = __shfl_xor(wk, o, kWave);
      const int oi = __shfl_xor(wi, o, kWave);
      if (key_before(ok, oi, wk, wi)) {
        wk = ok;
        wi = oi;
      }
    }
    // candidate ids are distinct, so exactly the lane whose best it was marks it taken
    if (bs >= 0 && bi == wi) taken |= 1u << bs;
    if (lane == j) {
      sel_key = wk;
      sel_idx = wi;
    }
  }
  // weights as select_topk: exp(key_j - key_0) over the kept keys, or over all E keys
  const float kmax = __shfl(sel_key, 0, kWave);
  const float num = (lane < k) ? expf(sel_key - kmax) : 0.0f;
  float den;
  if (renormalize) {
    den = wave_sum(num);
  } else {
    float zs = 0.0f;
    if (lane < n_slices) {
      const float2 st = stats[static_cast<size_t>(t) * n_slices + lane];
      if (st.x != -INFINITY) zs = st.y * expf(st.x - kmax);
    }
    den = wave_sum(zs);
  }
  if (lane < k) {
    int32_t* out = packed + static_cast<size_t>(t) * 2 * k;
    out[lane] = sel_idx;
    out[k + lane] = __float_as_int(num / den);
  }
}

template <int EL, int TB, int NFW>
hipError_t launch_slices(const void* x, const void* w_router, const float* bias, int T, int D, int E, int k,
                         float* logits_out, float* cand_key, int32_t* cand_id, float2* stats, hipStream_t stream) {
  constexpr int SW = 4 * NFW * 16;
  const int n_slices = (E + SW - 1) / SW;
  const dim3 grid(n_slices * ((T + TB - 1) / TB));
  // small batches split D over 4 wave groups (16 waves per workgroup) when the row holds
  // 4 x 256 bytes; otherwise the longest K block (512, 256 or 128 bytes) that divides the row
  const int row_bytes = D * ElSize<EL>::v;
  if constexpr (TB == 16) {
    if (row_bytes % 1024 == 0) {
      hipLaunchKernelGGL((router_slice_kernel<EL, TB, NFW, 4, 4>), grid, dim3(1024), 0, stream, x, w_router, bias,
                         T, D, E, k, n_slices, logits_out, cand_key, cand_id, stats);
      return hipGetLastError();
    }
  }
  if (row_bytes % 512 == 0)
    hipLaunchKernelGGL((router_slice_kernel<EL, TB, NFW, 8 / NFW, 1>), grid, dim3(256), 0, stream, x, w_router,
                       bias, T, D, E, k, n_slices, logits_out, cand_key, cand_id, stats);
  else if (row_bytes % 256 == 0)
    hipLaunchKernelGGL((router_slice_kernel<EL, TB, NFW, 4, 1>), grid, dim3(256), 0, stream, x, w_router, bias, T,
                       D, E, k, n_slices, logits_out, cand_key, cand_id, stats);
  else
    hipLaunchKernelGGL((router_slice_kernel<EL, TB, NFW, 2, 1>), grid, dim3(256), 0, stream, x, w_router, bias, T,
                       D, E, k, n_slices, logits_out, cand_key, cand_id, stats);
  return hipGetLastError();
}

}  // namespace

int router_fused_slices(int T, int E) {
  const int sw = T <= kFusedSmallT ? 64 : 128;
  return (E + sw - 1) / sw;
}

hipError_t launch_router_topk(int el, const void* x, const void* w_router, const float* bias, int T, int D, int E,
                              int k, int renormalize, float* logits_out, int32_t* packed, float* cand_key,
                              int32_t* cand_id, float2* stats, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  hipError_t e;
  // small batches: 16-token blocks and 64-expert slices (E / 64 * T / 16 workgroups);
  // larger ones: 64-token blocks and 128-expert slices (fewer re-reads of x and W_r)
  if (T <= kFusedSmallT)
    e = el == EL_BF16 ? launch_slices<EL_BF16, 16, 1>(x, w_router, bias, T, D, E, k, logits_out, cand_key, cand_id,
                                                       stats, stream)
                      : launch_slices<EL_F32, 16, 1>(x, w_router, bias, T, D, E, k, logits_out, cand_key, cand_id,
                                                      stats, stream);
  else
    e = el == EL_BF16 ? launch_slices<EL_BF16, 64, 2>(x, w_router, bias, T, D, E, k, logits_out, cand_key, cand_id,
                                                       stats, stream)
                      : launch_slices<EL_F32, 64, 2>(x, w_router, bias, T, D, E, k, logits_out, cand_key, cand_id,
                                                      stats, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(router_merge_kernel, dim3((T + 3) / 4), dim3(256), 0, stream, cand_key, cand_id, stats, T, E,
                     k, router_fused_slices(T, E), renormalize, packed);
  return hipGetLastError();
}

}  // namespace moe
