// Top-k selection of one token's experts by one wave64, shared by the routing kernels.
//
// Source: the router of "Tối ưu hóa mô hình Qwen 3.5-397B MoE trên hạ tầng TPU Ironwood",
// section "3. Sparse Mixture-of-Experts (MoE)" (softmax distribution, top 10 of 512), and
// the packed id/weight blob of "Systems Engineering Playbook: Qwen 3.5 MoE on Ironwood
// TPU", section "Fusing Three Collectives Into Two".
//
// Lane l holds the fp32 keys of experts l, l + 64, l + 128, ... (key[i] is expert
// l + 64 i).  Each of the k rounds takes every lane's best not-yet-taken key and reduces
// the (key, index) pairs across the wave with the order "larger key first, then lower
// index", so equal keys (and -0.0 vs +0.0) go to the lower expert id.  The weights are a
// softmax over the kept keys (the renormalised top-k of the full softmax, whose
// denominator cancels), or over all E keys when renormalisation is off.
#pragma once

#include "common.hpp"

namespace moe {

constexpr int kMaxKeysPerLane = 16;  // E <= 16 * 64

// a before b in the selection order.
__device__ __forceinline__ bool key_before(float ka, int ia, float kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}

// key[i] for i < PL: keys as above; entries of experts >= E are ignored.  Writes the
// token's ids to out[0..k) and the weights' bits to out[k..2k).
template <int PL>
__device__ __forceinline__ void select_topk(const float (&key)[PL], int E, int k, int renormalize,
                                            int32_t* __restrict__ out) {
  const int lane = lane_id();
  uint32_t taken = 0;  // bit i: expert lane + 64 i already selected (or does not exist)
#pragma unroll
  for (int i = 0; i < PL; ++i)
    if (lane + i * kWave >= E) taken |= 1u << i;

  float sel_key = 0.0f;  // lane j < k keeps the j-th selected key and id
  int sel_idx = 0;
  for (int j = 0; j < k; ++j) {
    // best not-taken candidate of this lane (sentinel: lowest priority possible)
    float bk = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const int e = lane + i * kWave;
      if (!((taken >> i) & 1u) && key_before(key[i], e, bk, bi)) {
        bk = key[i];
        bi = e;
      }
    }
    // wave-wide arg-best
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ok = __shfl_xor(bk, o, kWave);
      const int oi = __shfl_xor(bi, o, kWave);
      if (key_before(ok, oi, bk, bi)) {
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
    for (int i = 0; i < PL; ++i)
      if (lane + i * kWave < E) s += expf(key[i] - kmax);
    den = wave_sum(s);
  }
  if (lane < k) {
    out[lane] = sel_idx;
    out[k + lane] = __float_as_int(num / den);
  }
}

}  // namespace moe
