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

// (bk, bi) <- the better of itself and the pair held by the lane that DPP control CTRL
// selects (a VALU operand modifier: no LDS round trip).
template <int CTRL>
__device__ __forceinline__ void dpp_best(float& bk, int& bi) {
  const float ok = __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(bk), __float_as_int(bk), CTRL, 0xF, 0xF,
                                                              false));
  const int oi = __builtin_amdgcn_update_dpp(bi, bi, CTRL, 0xF, 0xF, false);
  if (key_before(ok, oi, bk, bi)) {
    bk = ok;
    bi = oi;
  }
}

// Wave-wide best (key, index) pair, returned to every lane.  Within each 16-lane row:
// quad exchanges (lane ^ 1, lane ^ 2), then the half-row mirror (lane i <-> 7 - i of each
// 8) and the row mirror (i <-> 15 - i), after which every lane of a row holds the row's
// best; the four row winners are then read out and compared.  The order is a strict
// total order on (key, index), so the result does not depend on the reduction's shape.
__device__ __forceinline__ void wave_best(float& bk, int& bi) {
  dpp_best<0xB1>(bk, bi);   // quad_perm [1, 0, 3, 2]
  dpp_best<0x4E>(bk, bi);   // quad_perm [2, 3, 0, 1]
  dpp_best<0x141>(bk, bi);  // row_half_mirror
  dpp_best<0x140>(bk, bi);  // row_mirror
  float rk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bk), 0));
  int ri = __builtin_amdgcn_readlane(bi, 0);
#pragma unroll
  for (int r = 1; r < 4; ++r) {
    const float ok = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bk), 16 * r));
    const int oi = __builtin_amdgcn_readlane(bi, 16 * r);
    if (key_before(ok, oi, rk, ri)) {
      rk = ok;
      ri = oi;
    }
  }
  bk = rk;
  bi = ri;
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
    wave_best(bk, bi);
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
