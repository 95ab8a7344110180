// Router selection: fp32 keys -> top-k experts and weights -> packed [T][2][k] blob.
//
// Source: the router of "Tối ưu hóa mô hình Qwen 3.5-397B MoE trên hạ tầng TPU Ironwood",
// section "3. Sparse Mixture-of-Experts (MoE)" (projection, softmax distribution,
// top 10 of 512), and the packed id/weight blob of "Systems Engineering Playbook:
// Qwen 3.5 MoE on Ironwood TPU", section "Fusing Three Collectives Into Two".
//
// One wave64 per token.  Lane l owns the keys of experts l, l + 64, l + 128, ...
// (at most 16 per lane, E <= 1024).  Each of the k rounds takes every lane's best
// not-yet-taken key and reduces the (key, index) pairs across the wave with the
// order "larger key first, then lower index", so equal keys (and -0.0 vs +0.0) go
// to the lower expert id.  The weights are a softmax over the kept keys (the
// renormalised top-k of the full softmax, whose denominator cancels), or over all E
// keys when renormalisation is off.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kMaxPerLane = 16;  // E <= 16 * 64

// a before b in the selection order.
__device__ __forceinline__ bool before(float ka, int ia, float kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}

// SPLIT: the router product arrives as n_parts > 1 partial sums over slices of D.
template <bool SPLIT>
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
  uint32_t taken = 0;  // bit i: expert lane + 64 i already selected (or does not exist)
  const int per_lane = (E + kWave - 1) / kWave;
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int e = lane + i * kWave;
    key[i] = -INFINITY;
    if (i < per_lane && e < E) {
      float v = row[e];
      if (!SPLIT && bias) v = v + bias[e];  // one fp32 add
      key[i] = v;
    } else {
      taken |= 1u << i;
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

  float sel_key = 0.0f;  // lane j < k keeps the j-th selected key and id
  int sel_idx = 0;
  for (int j = 0; j < k; ++j) {
    // best not-taken candidate of this lane (sentinel: lowest priority possible)
    float bk = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      const int e = lane + i * kWave;
      if (!((taken >> i) & 1u) && before(key[i], e, bk, bi)) {
        bk = key[i];
        bi = e;
      }
    }
    // wave-wide arg-best
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ok = __shfl_xor(bk, o, kWave);
      const int oi = __shfl_xor(bi, o, kWave);
      if (before(ok, oi, bk, bi)) {
        bk = ok;
        bi = oi;
      }
    }
    if (bi < E && (bi & (kWave - 1)) == lane) taken |= 1u << (bi / kWave);
    if (lane == j) {
      sel_key = bk;
      sel_idx = bi;
    }
  }

  // Weights: exp(key_j - key_0) over the kept keys (or all keys), fp32.
  const float kmax = __shfl(sel_key, 0, kWave);
  const float num = (lane < k) ? expf(sel_key - kmax) : 0.0f;
  float den;
  if (renormalize) {
    den = wave_sum(num);
  } else {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      const int e = lane + i * kWave;
      if (i < per_lane && e < E) s += expf(key[i] - kmax);
    }
    den = wave_sum(s);
  }
  if (lane < k) {
    const float w = num / den;
    int32_t* out = packed + static_cast<size_t>(t) * 2 * k;
    out[lane] = sel_idx;
    out[k + lane] = __float_as_int(w);
  }
}

}  // namespace

hipError_t launch_route(const float* parts, int n_parts, float* logits, const float* bias, int T, int E, int k,
                        int renormalize, int32_t* packed, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int waves_per_block = 4;
  dim3 grid((T + waves_per_block - 1) / waves_per_block);
  if (n_parts > 1)
    hipLaunchKernelGGL(route_kernel<true>, grid, dim3(waves_per_block * kWave), 0, stream, parts, n_parts, logits,
                       bias, T, E, k, renormalize, packed);
  else
    hipLaunchKernelGGL(route_kernel<false>, grid, dim3(waves_per_block * kWave), 0, stream, parts, n_parts, logits,
                       bias, T, E, k, renormalize, packed);
  return hipGetLastError();
}

}  // namespace moe
