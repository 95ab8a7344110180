// Fused router: projection, top-k, weights and the packed blob in one kernel, so the
// [T][E] logits never have to go through HBM.
//
// Source: the router of "Tối ưu hóa mô hình Qwen 3.5-397B MoE trên hạ tầng TPU Ironwood",
// section "3. Sparse Mixture-of-Experts (MoE)" (projection to the experts, softmax
// distribution, top 10 of 512); fusing the selection into the kernel that produces the
// logits is the open item of "Systems Engineering Playbook: Qwen 3.5 MoE on Ironwood
// TPU", section "The Remaining Roadmap"; routing needs full-precision accumulation
// (Playbook, "Roofline Validation").
//
// One 256-thread workgroup owns 64 tokens and every expert (E <= 512): wave w computes
// logits[t][e] for experts 128 w .. 128 w + 127 of all 64 tokens with 16x16 MFMAs (fp32
// accumulation), W_r rows streaming from L2 into registers as the A operand, the token
// rows staged in LDS per K block as the B operand (as in the grouped GEMM).  The 64 x E
// fp32 logits then go to LDS, and each wave routes 16 of the tokens with select_topk
// (the same selection code as the unfused path), optionally copying the logits rows out.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "kernels.hpp"
#include "topk.hpp"

namespace moe {

namespace {

constexpr int kTok = 64;                  // tokens per workgroup
constexpr int kMF = kTok / 16;            // 16-token B fragments
constexpr int kNFW = 8;                   // 16-expert A fragments per wave (128 experts)
constexpr int kKSteps = 2;                // 64-byte K steps per block
constexpr int kKBlk = kKSteps * 64;       // bytes of each row per K block
constexpr int kRow = kKBlk + 16;          // padded LDS row of the token tile (bytes)
constexpr int kLogRow = kMaxFusedExperts + 4;  // padded LDS row of the logits tile (floats)
constexpr int kTokBytes = 2 * kTok * kRow;
constexpr int kLogBytes = kTok * kLogRow * 4;
constexpr int kLdsBytes = kTokBytes > kLogBytes ? kTokBytes : kLogBytes;

template <int EL>
__global__ __launch_bounds__(256, 1) void router_topk_kernel(const void* __restrict__ x,
                                                             const void* __restrict__ w_router,
                                                             const float* __restrict__ bias, int T, int D, int E,
                                                             int k, int renormalize, float* __restrict__ logits_out,
                                                             int32_t* __restrict__ packed) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];
  constexpr int ES = ElSize<EL>::v;
  const int t0 = blockIdx.x * kTok;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave, lrow = lane & 15, lgrp = lane >> 4;
  const uint32_t row_bytes = static_cast<uint32_t>(D) * ES;
  const int nblk = static_cast<int>(row_bytes / kKBlk);

  // operand offsets: W_r rows past E and token rows past T re-read the last valid row
  // (their results are never used)
  const __amdgpu_buffer_rsrc_t wres = buffer_rsrc(w_router);
  const __amdgpu_buffer_rsrc_t xres = buffer_rsrc(x);
  uint32_t woff[kNFW];
#pragma unroll
  for (int nf = 0; nf < kNFW; ++nf) {
    const int e = min(wv * kNFW * 16 + nf * 16 + lrow, E - 1);
    woff[nf] = static_cast<uint32_t>(e) * row_bytes + lgrp * 16;
  }
  constexpr int kCpr = kKBlk / 16;         // 16-byte chunks per token row per block
  constexpr int kRpp = 256 / kCpr;         // token rows per pass
  constexpr int kPasses = kTok / kRpp;
  const int crow = threadIdx.x / kCpr, ccol = (threadIdx.x % kCpr) * 16;
  uint32_t toff[kPasses];
#pragma unroll
  for (int i = 0; i < kPasses; ++i) {
    const int t = min(t0 + crow + i * kRpp, T - 1);
    toff[i] = static_cast<uint32_t>(t) * row_bytes + ccol;
  }

  f32x4 acc[kNFW][kMF];
#pragma unroll
  for (int nf = 0; nf < kNFW; ++nf)
#pragma unroll
    for (int mf = 0; mf < kMF; ++mf) acc[nf][mf] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 wr[2][kNFW][kKSteps];
  u32x4 tv[kPasses];
  auto ld_w = [&](u32x4 (&w)[kNFW][kKSteps], int kb) {
    const uint32_t o = static_cast<uint32_t>(min(kb, nblk - 1)) * kKBlk;
#pragma unroll
    for (int st = 0; st < kKSteps; ++st)
#pragma unroll
      for (int nf = 0; nf < kNFW; ++nf) w[nf][st] = buffer_load16(wres, woff[nf], o + st * 64);
  };
  auto ld_t = [&](int kb) {
    const uint32_t o = static_cast<uint32_t>(min(kb, nblk - 1)) * kKBlk;
#pragma unroll
    for (int i = 0; i < kPasses; ++i) tv[i] = buffer_load16(xres, toff[i], o);
  };
  auto st_t = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kPasses; ++i)
      *reinterpret_cast<u32x4*>(&lds[buf * kTok * kRow + (crow + i * kRpp) * kRow + ccol]) = tv[i];
  };
  auto mm = [&](const u32x4 (&w)[kNFW][kKSteps], int buf) {
    const uint8_t* sb = &lds[buf * kTok * kRow + lrow * kRow + lgrp * 16];
#pragma unroll
    for (int st = 0; st < kKSteps; ++st)
#pragma unroll
      for (int mf = 0; mf < kMF; ++mf) {
        const u32x4 b = *reinterpret_cast<const u32x4*>(sb + mf * 16 * kRow + st * 64);
#pragma unroll
        for (int nf = 0; nf < kNFW; ++nf) acc[nf][mf] = mfma_chunk<EL>(w[nf][st], b, acc[nf][mf]);
      }
  };

  // K blocks: weights one block ahead in a two-block register ring, token rows one
  // block ahead through registers into the other LDS buffer
  ld_t(0);
  ld_w(wr[0], 0);
  st_t(0);
  __syncthreads();
  for (int kb = 0; kb < nblk; kb += 2) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (j > 0 && kb + j >= nblk) break;
      ld_t(kb + j + 1);
      ld_w(wr[(j + 1) & 1], kb + j + 1);
      mm(wr[j], (kb + j) & 1);
      st_t((kb + j + 1) & 1);
      __syncthreads();
    }
  }

  // logits tile to LDS: lane holds experts 4 (l / 16) + r of each fragment for token l % 16
  float* lt = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int nf = 0; nf < kNFW; ++nf)
#pragma unroll
    for (int mf = 0; mf < kMF; ++mf) {
      const int e = wv * kNFW * 16 + nf * 16 + lgrp * 4;
      *reinterpret_cast<f32x4*>(&lt[(mf * 16 + lrow) * kLogRow + e]) = acc[nf][mf];
    }
  __syncthreads();

  // route 16 tokens per wave
  constexpr int PL = kMaxFusedExperts / kWave;
  for (int r = wv; r < kTok; r += 4) {
    const int t = t0 + r;
    if (t >= T) break;
    float key[PL];
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const int e = lane + i * kWave;
      key[i] = -INFINITY;
      if (e < E) {
        const float v = lt[r * kLogRow + e];
        if (logits_out) logits_out[static_cast<size_t>(t) * E + e] = v;
        key[i] = bias ? v + bias[e] : v;  // one fp32 add
      }
    }
    select_topk(key, E, k, renormalize, packed + static_cast<size_t>(t) * 2 * k);
  }
}

}  // namespace

hipError_t launch_router_topk(int el, const void* x, const void* w_router, const float* bias, int T, int D, int E,
                              int k, int renormalize, float* logits_out, int32_t* packed, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const dim3 grid((T + kTok - 1) / kTok);
  if (el == EL_BF16)
    hipLaunchKernelGGL(router_topk_kernel<EL_BF16>, grid, dim3(256), 0, stream, x, w_router, bias, T, D, E, k,
                       renormalize, logits_out, packed);
  else
    hipLaunchKernelGGL(router_topk_kernel<EL_F32>, grid, dim3(256), 0, stream, x, w_router, bias, T, D, E, k,
                       renormalize, logits_out, packed);
  return hipGetLastError();
}

}  // namespace moe
