// Runtime numerical audit: an fp32 shadow of the layer on sampled tokens.
//
// Source: the "Numerical Verification Layer" of "Systems Engineering Playbook: Qwen 3.5
// MoE on Ironwood TPU" (section "Roofline Validation": low-precision paths are checked
// against a high-precision evaluation, because routing and FP8 scaling are sensitive to
// accumulation precision).
//
// For each sampled token t the shadow evaluates, from the stored tensors and in fp32:
//   ref[t] = sum_j w[t][j] * W_down,e (silu(W_gate,e x_t) * (W_up,e x_t))   (local slots)
//            + W_down,s (silu(W_gate,s x_t) * (W_up,s x_t))                (shared expert)
// with E4M3 weights decoded and multiplied by their per-channel scales, but x and h
// never quantised, so it measures what the fast path's rounding and quantisation cost.
// The routing (ids and weights) is taken from the packed blob the layer used.  Then
// max_t,d |y[t][d] - ref[t][d]| and max_t,d |ref[t][d]| go to result[0], result[1].
//
// Work items are (sample, slot), slot top_k being the shared expert.  One workgroup per
// item; each wave forms one dot product at a time, its lanes reading 16-byte chunks of
// a weight row (coalesced for row-major weights, whole 1 KB runs for packed ones) and
// the fp32 vector from LDS.  Not a hot path: a few hundred microseconds for 16 tokens.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

struct AuditArgs {
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
  float* h;        // [items][i_max]
  float* out;      // [items][D]
  float* stats;    // [n_sample][2]
  float* ref_out;  // [n_sample][D] or NULL
  float* result;   // [2]
  int i_max;
};

__device__ __forceinline__ int elem_bytes(int el) { return el == EL_F32 ? 4 : el == EL_BF16 ? 2 : 1; }

__device__ __forceinline__ float load_act(const void* p, size_t i, int el) {
  if (el == EL_F32) return static_cast<const float*>(p)[i];
  return bf16_bits_to_f32(static_cast<const uint16_t*>(p)[i]);
}

// Byte offset of 16-byte chunk c of row r of a [rows][row_bytes] matrix in either layout.
__device__ __forceinline__ size_t chunk_offset(int r, int c, int row_bytes, bool packed) {
  if (!packed) return static_cast<size_t>(r) * row_bytes + static_cast<size_t>(c) * 16;
  const size_t run = static_cast<size_t>(r / 16) * (row_bytes / 64) + c / 4;
  return (run * 64 + (r % 16) + 16 * (c % 4)) * 16;
}

// sum_i row[i] * v[i] over n elements of row r, by one wave (v in LDS, fp32).
__device__ float row_dot(const uint8_t* m, int r, int n, int el, bool packed, const float* v) {
  const int row_bytes = n * elem_bytes(el);
  const int chunks = row_bytes / 16;
  float s = 0.0f;
  for (int c = lane_id(); c < chunks; c += kWave) {
    const u32x4 q = *reinterpret_cast<const u32x4*>(m + chunk_offset(r, c, row_bytes, packed));
    const uint32_t w4[4] = {q.x, q.y, q.z, q.w};
    if (el == EL_F32) {
#pragma unroll
      for (int i = 0; i < 4; ++i) s = fmaf(__uint_as_float(w4[i]), v[c * 4 + i], s);
    } else if (el == EL_BF16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s = fmaf(bf16_bits_to_f32(w4[i] & 0xFFFFu), v[c * 8 + 2 * i], s);
        s = fmaf(bf16_bits_to_f32(w4[i] >> 16), v[c * 8 + 2 * i + 1], s);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w4[i]), false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w4[i]), true);
        s = fmaf(lo[0], v[c * 16 + 4 * i], s);
        s = fmaf(lo[1], v[c * 16 + 4 * i + 1], s);
        s = fmaf(hi[0], v[c * 16 + 4 * i + 2], s);
        s = fmaf(hi[1], v[c * 16 + 4 * i + 3], s);
      }
    }
  }
  return wave_sum(s);
}

// The expert of item (s, j): matrices, element type, rows; false if the slot is not local
// (or there is no shared expert).
struct ItemExpert {
  const uint8_t *g, *u, *d;
  const float *sg, *su, *sd;
  int rows, el;
};

__device__ bool item_expert(const AuditArgs& a, int s, int j, ItemExpert& ex) {
  const int t = min(max(a.sample[s], 0), a.T - 1);
  if (j == a.k) {
    if (a.I_shared == 0 || !a.sh_gate) return false;
    ex = {static_cast<const uint8_t*>(a.sh_gate), static_cast<const uint8_t*>(a.sh_up),
          static_cast<const uint8_t*>(a.sh_down), nullptr, nullptr, nullptr, a.I_shared, a.act_el};
    return true;
  }
  const int e = a.packed[static_cast<size_t>(t) * 2 * a.k + j] - a.e_begin;
  if (e < 0 || e >= a.n_local) return false;
  const size_t mat = static_cast<size_t>(a.I) * a.D * elem_bytes(a.w_el);
  const bool sc = a.w_el == EL_E4M3;
  ex = {static_cast<const uint8_t*>(a.w_gate) + e * mat, static_cast<const uint8_t*>(a.w_up) + e * mat,
        static_cast<const uint8_t*>(a.w_down) + e * mat, sc ? a.s_gate + static_cast<size_t>(e) * a.I : nullptr,
        sc ? a.s_up + static_cast<size_t>(e) * a.I : nullptr, sc ? a.s_down + static_cast<size_t>(e) * a.D : nullptr,
        a.I, a.w_el};
  return true;
}

__global__ __launch_bounds__(256) void audit_h_kernel(AuditArgs a) {
  extern __shared__ float vec[];  // x_t, D floats
  const int item = blockIdx.x, s = item / (a.k + 1), j = item % (a.k + 1);
  float* h = a.h + static_cast<size_t>(item) * a.i_max;
  ItemExpert ex;
  if (!item_expert(a, s, j, ex)) return;  // uniform over the workgroup
  const int t = min(max(a.sample[s], 0), a.T - 1);
  for (int i = threadIdx.x; i < a.D; i += blockDim.x)
    vec[i] = load_act(a.x, static_cast<size_t>(t) * a.D + i, a.act_el);
  __syncthreads();
  const bool pk = a.packed_layout != 0;
  for (int r = threadIdx.x / kWave; r < ex.rows; r += blockDim.x / kWave) {
    float g = row_dot(ex.g, r, a.D, ex.el, pk, vec);
    float u = row_dot(ex.u, r, a.D, ex.el, pk, vec);
    if (ex.sg) {
      g *= ex.sg[r];
      u *= ex.su[r];
    }
    if (lane_id() == 0) h[r] = g / (1.0f + expf(-g)) * u;
  }
}

__global__ __launch_bounds__(256) void audit_out_kernel(AuditArgs a) {
  extern __shared__ float vec[];  // h of the item
  const int item = blockIdx.x, s = item / (a.k + 1), j = item % (a.k + 1);
  float* out = a.out + static_cast<size_t>(item) * a.D;
  ItemExpert ex;
  if (!item_expert(a, s, j, ex)) return;
  const float* h = a.h + static_cast<size_t>(item) * a.i_max;
  for (int i = threadIdx.x; i < ex.rows; i += blockDim.x) vec[i] = h[i];
  __syncthreads();
  const bool pk = a.packed_layout != 0;
  for (int r = threadIdx.x / kWave; r < a.D; r += blockDim.x / kWave) {
    float o = row_dot(ex.d, r, ex.rows, ex.el, pk, vec);
    if (ex.sd) o *= ex.sd[r];
    if (lane_id() == 0) out[r] = o;
  }
}

// One workgroup per sample: the reference row in slot order (shared expert last), its
// distance to y, per-sample maxima.
__global__ __launch_bounds__(256) void audit_combine_kernel(AuditArgs a) {
  __shared__ float red[2][256];
  __shared__ float w[33];  // slot weight, 0 for a slot that is not local (top_k <= 32, + shared)
  const int s = blockIdx.x;
  const int t = min(max(a.sample[s], 0), a.T - 1);
  if (threadIdx.x <= a.k) {
    const int j = threadIdx.x;
    ItemExpert ex;
    const bool live = item_expert(a, s, j, ex);
    w[j] = !live ? 0.0f : j < a.k ? __int_as_float(a.packed[static_cast<size_t>(t) * 2 * a.k + a.k + j]) : 1.0f;
  }
  __syncthreads();
  float md = 0.0f, mr = 0.0f;
  for (int d = threadIdx.x; d < a.D; d += blockDim.x) {
    float ref = 0.0f;
    for (int j = 0; j < a.k; ++j)
      if (w[j] != 0.0f) ref = fmaf(w[j], a.out[(static_cast<size_t>(s) * (a.k + 1) + j) * a.D + d], ref);
    if (w[a.k] != 0.0f) ref += a.out[(static_cast<size_t>(s) * (a.k + 1) + a.k) * a.D + d];
    const float yv = load_act(a.y, static_cast<size_t>(t) * a.D + d, a.out_el);
    md = fmaxf(md, fabsf(yv - ref));
    mr = fmaxf(mr, fabsf(ref));
    if (a.ref_out) a.ref_out[static_cast<size_t>(s) * a.D + d] = ref;
  }
  red[0][threadIdx.x] = md;
  red[1][threadIdx.x] = mr;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) {
      red[0][threadIdx.x] = fmaxf(red[0][threadIdx.x], red[0][threadIdx.x + o]);
      red[1][threadIdx.x] = fmaxf(red[1][threadIdx.x], red[1][threadIdx.x + o]);
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    a.stats[2 * s] = red[0][0];
    a.stats[2 * s + 1] = red[1][0];
  }
}

__global__ __launch_bounds__(256) void audit_reduce_kernel(AuditArgs a) {
  __shared__ float red[2][256];
  float md = 0.0f, mr = 0.0f;
  for (int s = threadIdx.x; s < a.n_sample; s += blockDim.x) {
    md = fmaxf(md, a.stats[2 * s]);
    mr = fmaxf(mr, a.stats[2 * s + 1]);
  }
  red[0][threadIdx.x] = md;
  red[1][threadIdx.x] = mr;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) {
      red[0][threadIdx.x] = fmaxf(red[0][threadIdx.x], red[0][threadIdx.x + o]);
      red[1][threadIdx.x] = fmaxf(red[1][threadIdx.x], red[1][threadIdx.x + o]);
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    a.result[0] = red[0][0];
    a.result[1] = red[1][0];
  }
}

}  // namespace

size_t audit_workspace_bytes(int n_sample, int k, int D, int i_max) {
  const size_t items = static_cast<size_t>(n_sample) * (k + 1);
  auto up = [](size_t b) { return (b + 255) / 256 * 256; };
  return up(items * i_max * 4) + up(items * static_cast<size_t>(D) * 4) + up(static_cast<size_t>(n_sample) * 8);
}

hipError_t launch_audit(const AuditLaunch& l, hipStream_t stream) {
  const int i_max = l.I > l.I_shared ? l.I : l.I_shared;
  const size_t items = static_cast<size_t>(l.n_sample) * (l.k + 1);
  auto up = [](size_t b) { return (b + 255) / 256 * 256; };
  uint8_t* ws = static_cast<uint8_t*>(l.ws);
  AuditArgs a;
  a.x = l.x; a.packed = l.packed; a.y = l.y; a.sample = l.sample;
  a.T = l.T; a.D = l.D; a.k = l.k; a.I = l.I; a.I_shared = l.I_shared; a.e_begin = l.e_begin;
  a.n_local = l.n_local; a.n_sample = l.n_sample;
  a.act_el = l.act_el; a.w_el = l.w_el; a.out_el = l.out_el; a.packed_layout = l.packed_layout;
  a.w_gate = l.w_gate; a.w_up = l.w_up; a.w_down = l.w_down; a.s_gate = l.s_gate; a.s_up = l.s_up;
  a.s_down = l.s_down; a.sh_gate = l.sh_gate; a.sh_up = l.sh_up; a.sh_down = l.sh_down;
  a.h = reinterpret_cast<float*>(ws);
  a.out = reinterpret_cast<float*>(ws + up(items * i_max * 4));
  a.stats = reinterpret_cast<float*>(ws + up(items * i_max * 4) + up(items * static_cast<size_t>(l.D) * 4));
  a.ref_out = l.ref_out;
  a.result = l.result;
  a.i_max = i_max;
  const dim3 grid_items(static_cast<unsigned>(items));
  hipLaunchKernelGGL(audit_h_kernel, grid_items, dim3(256), l.D * sizeof(float), stream, a);
  hipLaunchKernelGGL(audit_out_kernel, grid_items, dim3(256), i_max * sizeof(float), stream, a);
  hipLaunchKernelGGL(audit_combine_kernel, dim3(l.n_sample), dim3(256), 0, stream, a);
  hipLaunchKernelGGL(audit_reduce_kernel, dim3(1), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace moe
