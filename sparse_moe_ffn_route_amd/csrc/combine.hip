// Unpermute + local reduction with the routing weights, plus the shared expert.
//
// Source: "unpermutation + local reduction" of "Systems Engineering Playbook: Qwen 3.5
// MoE on Ironwood TPU" (table "Three High-Leverage Optimizations"); the always-on
// shared expert of "Tối ưu hóa mô hình Qwen 3.5-397B MoE trên hạ tầng TPU Ironwood",
// section "3. Sparse Mixture-of-Experts (MoE)" (added with weight one: the page's
// formula is missing).
//
//   y[t] = sum_j w[t][j] * out_rows[inv_pos[t][j]]  (slots with inv_pos < 0 skipped)
//          + shared_out[t]
// in fp32, slot order, shared row last, one rounding to the output type.
// One wave per (token, 512-column chunk); each lane owns 8 consecutive columns, so
// every source row is read as 16-byte (bf16) or 32-byte (fp32) coalesced pieces.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

template <int OUT>
__device__ __forceinline__ void load8(const void* base, size_t idx, float v[8]) {
  if (OUT == EL_BF16) {
    const uint4 p = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + idx);
    const uint32_t w[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = bf16_bits_to_f32(w[q] & 0xFFFFu);
      v[2 * q + 1] = bf16_bits_to_f32(w[q] >> 16);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + idx);
    const float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

template <int OUT>
__device__ __forceinline__ void store8(void* base, size_t idx, const float v[8]) {
  if (OUT == EL_BF16) {
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) w[q] = bf16x2_bits(v[2 * q], v[2 * q + 1]);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + idx) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(base) + idx);
    p[0] = make_float4(v[0], v[1], v[2], v[3]);
    p[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
}

template <int OUT>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ out_rows,
                                                      const int32_t* __restrict__ packed,
                                                      const int32_t* __restrict__ inv_pos,
                                                      const void* __restrict__ shared_out, int T, int D, int k,
                                                      int chunks, void* __restrict__ y) {
  const int wid = blockIdx.x * 4 + threadIdx.x / kWave;
  const int lane = lane_id();
  const int t = wid / chunks;
  if (t >= T) return;
  const int col = (wid % chunks) * 512 + lane * 8;
  if (col >= D) return;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const int32_t* wbits = packed + static_cast<size_t>(t) * 2 * k + k;
  for (int j = 0; j < k; ++j) {
    const int r = inv_pos[static_cast<size_t>(t) * k + j];
    if (r < 0) continue;
    const float w = __int_as_float(wbits[j]);
    float v[8];
    load8<OUT>(out_rows, static_cast<size_t>(r) * D + col, v);
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = fmaf(w, v[q], acc[q]);
  }
  if (shared_out) {
    float v[8];
    load8<OUT>(shared_out, static_cast<size_t>(t) * D + col, v);
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] += v[q];
  }
  store8<OUT>(y, static_cast<size_t>(t) * D + col, acc);
}

}  // namespace

hipError_t launch_combine(int out_el, const void* out_rows, const int32_t* packed, const int32_t* inv_pos,
                          const void* shared_out, int T, int D, int k, void* y, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int chunks = (D + 511) / 512;
  const int waves = T * chunks;
  dim3 grid((waves + 3) / 4);
  if (out_el == EL_BF16)
    hipLaunchKernelGGL(combine_kernel<EL_BF16>, grid, dim3(256), 0, stream, out_rows, packed, inv_pos, shared_out,
                       T, D, k, chunks, y);
  else
    hipLaunchKernelGGL(combine_kernel<EL_F32>, grid, dim3(256), 0, stream, out_rows, packed, inv_pos, shared_out,
                       T, D, k, chunks, y);
  return hipGetLastError();
}

}  // namespace moe
