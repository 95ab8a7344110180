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
// every source row is read as 16-byte (bf16) or 32-byte (fp32) coalesced pieces.  The
// slots are taken in batches of 8: all of a batch's row loads (and the shared row) are
// issued before the first is summed, so a wave keeps up to 9 row pieces in flight; the
// sum itself still runs in slot order.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

// Raw 8-column piece: 16 bytes of bf16 or 32 bytes of fp32, converted when summed.
template <int OUT> struct Piece;
template <> struct Piece<EL_BF16> { uint4 a; };
template <> struct Piece<EL_F32> { float4 a, b; };

// The piece at byte offset voff of one row, read through that row's buffer resource
// (an empty resource reads zeros and touches no memory).
template <int OUT>
__device__ __forceinline__ Piece<OUT> load_piece(__amdgpu_buffer_rsrc_t row, uint32_t voff) {
  Piece<OUT> p;
  if constexpr (OUT == EL_BF16) {
    p.a = __builtin_bit_cast(uint4, buffer_load16(row, voff, 0));
  } else {
    p.a = __builtin_bit_cast(float4, buffer_load16(row, voff, 0));
    p.b = __builtin_bit_cast(float4, buffer_load16(row, voff, 16));
  }
  return p;
}

template <int OUT>
__device__ __forceinline__ void unpack8(const Piece<OUT>& p, float v[8]) {
  if constexpr (OUT == EL_BF16) {
    const uint32_t w[4] = {p.a.x, p.a.y, p.a.z, p.a.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = bf16_bits_to_f32(w[q] & 0xFFFFu);
      v[2 * q + 1] = bf16_bits_to_f32(w[q] >> 16);
    }
  } else {
    v[0] = p.a.x; v[1] = p.a.y; v[2] = p.a.z; v[3] = p.a.w;
    v[4] = p.b.x; v[5] = p.b.y; v[6] = p.b.z; v[7] = p.b.w;
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
  constexpr int kBatch = 8;
  // wave-uniform by construction; readfirstlane lets the slot metadata load as scalars
  const int wid = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + threadIdx.x / kWave);
  const int lane = lane_id();
  const int t = wid / chunks;
  if (t >= T) return;
  const int col = (wid % chunks) * 512 + lane * 8;
  if (col >= D) return;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const int32_t* wbits = packed + static_cast<size_t>(t) * 2 * k + k;
  const int32_t* rows = inv_pos + static_cast<size_t>(t) * k;
  // Branch-free issue: every row is read through a resource of its own, and a missing
  // row (no shared expert, a slot without a local row, a slot past k) gets the empty
  // resource, so its load reads zeros without a memory access and is skipped in the sum.
  constexpr int kEs = OUT == EL_BF16 ? 2 : 4;
  const uint32_t voff = static_cast<uint32_t>(col) * kEs;
  const size_t row_bytes = static_cast<size_t>(D) * kEs;
  const Piece<OUT> sh = load_piece<OUT>(
      shared_out ? buffer_rsrc(static_cast<const uint8_t*>(shared_out) + static_cast<size_t>(t) * row_bytes)
                 : buffer_rsrc_empty(),
      voff);
  for (int j0 = 0; j0 < k; j0 += kBatch) {
    int r[kBatch];
    Piece<OUT> pc[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int rr = rows[min(j0 + u, k - 1)];
      r[u] = j0 + u < k ? rr : -1;
    }
    __builtin_amdgcn_sched_barrier(0);  // all of the batch's indices before its row loads
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const __amdgpu_buffer_rsrc_t res =
          r[u] >= 0 ? buffer_rsrc(static_cast<const uint8_t*>(out_rows) + static_cast<size_t>(r[u]) * row_bytes)
                    : buffer_rsrc_empty();
      pc[u] = load_piece<OUT>(res, voff);
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (r[u] < 0) continue;
      const float w = __int_as_float(wbits[j0 + u]);
      float v[8];
      unpack8<OUT>(pc[u], v);
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = fmaf(w, v[q], acc[q]);
    }
  }
  if (shared_out) {
    float v[8];
    unpack8<OUT>(sh, v);
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
