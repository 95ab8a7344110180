// Router selection: fp32 keys -> top-k experts and weights -> packed [T][2][k] blob.
//
// Source: the router of "Tối ưu hóa mô hình Qwen 3.5-397B MoE trên hạ tầng TPU Ironwood",
// section "3. Sparse Mixture-of-Experts (MoE)" (projection, softmax distribution,
// top 10 of 512), and the packed id/weight blob of "Systems Engineering Playbook:
// Qwen 3.5 MoE on Ironwood TPU", section "Fusing Three Collectives Into Two".
//
// One wave64 per token; the selection itself is select_topk (topk.hpp).
#include "common.hpp"
#include "kernels.hpp"
#include "topk.hpp"

namespace moe {

namespace {

// SPLIT: the router product arrives as n_parts > 1 partial sums over slices of D.
// kMaxPerLane: keys per lane (E <= 64 * kMaxPerLane).
template <bool SPLIT, int kMaxPerLane>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ parts, int n_parts,
                                                    float* __restrict__ logits, const float* __restrict__ bias,
                                                    int T, int E, int k, int renormalize,
                                                    int32_t* __restrict__ packed) {
  const int lane = lane_id();
  const int t = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (t >= T) return;
  const size_t part_stride = static_cast<size_t>(T) * E;
  const float* row = (SPLIT ? parts : logits) + static_cast<size_t>(t) * E;

  float key[kMaxPerLane];
  const int per_lane = (E + kWave - 1) / kWave;
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int e = lane + i * kWave;
    key[i] = -INFINITY;
    if (i < per_lane && e < E) {
      float v = row[e];
      if (!SPLIT && bias) v = v + bias[e];  // one fp32 add
      key[i] = v;
    }
  }
  if (SPLIT) {
    // add the partials in a fixed order; each partial's loads are issued together, so
    // the sum costs one memory latency per partial
#pragma unroll 1
    for (int p = 1; p < n_parts; ++p) {
      const float* prow = row + p * part_stride;
      float v[kMaxPerLane];
#pragma unroll
      for (int i = 0; i < kMaxPerLane; ++i) {
        const int e = lane + i * kWave;
        v[i] = (i < per_lane && e < E) ? prow[e] : 0.0f;
      }
#pragma unroll
      for (int i = 0; i < kMaxPerLane; ++i) key[i] += v[i];
    }
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      const int e = lane + i * kWave;
      if (i < per_lane && e < E) {
        logits[static_cast<size_t>(t) * E + e] = key[i];
        if (bias) key[i] = key[i] + bias[e];  // one fp32 add
      }
    }
  }

  select_topk(key, E, k, renormalize, packed + static_cast<size_t>(t) * 2 * k);
}

}  // namespace

hipError_t launch_route(const float* parts, int n_parts, float* logits, const float* bias, int T, int E, int k,
                        int renormalize, int32_t* packed, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int waves_per_block = 4;
  dim3 grid((T + waves_per_block - 1) / waves_per_block);
  const dim3 block(waves_per_block * kWave);
  // keys per lane: 8 cover up to 512 experts, kMaxKeysPerLane the largest E accepted
  if (E <= 8 * kWave) {
    if (n_parts > 1)
      hipLaunchKernelGGL((route_kernel<true, 8>), grid, block, 0, stream, parts, n_parts, logits, bias, T, E, k,
                         renormalize, packed);
    else
      hipLaunchKernelGGL((route_kernel<false, 8>), grid, block, 0, stream, parts, n_parts, logits, bias, T, E, k,
                         renormalize, packed);
  } else {
    if (n_parts > 1)
      hipLaunchKernelGGL((route_kernel<true, kMaxKeysPerLane>), grid, block, 0, stream, parts, n_parts, logits, bias,
                         T, E, k, renormalize, packed);
    else
      hipLaunchKernelGGL((route_kernel<false, kMaxKeysPerLane>), grid, block, 0, stream, parts, n_parts, logits, bias,
                         T, E, k, renormalize, packed);
  }
  return hipGetLastError();
}

}  // namespace moe
