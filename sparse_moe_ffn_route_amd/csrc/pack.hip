// Weight repacking, and a plain streaming-read kernel for measuring achievable HBM
// bandwidth on the running device.
//
// One-time repacking of weight matrices into the fragment-major order the grouped GEMM
// streams (see moe_pack_weights in moe.h): for output-row fragment f (16 rows) and
// 64-byte reduction slice s, bytes [s*64, s*64+64) of rows 16f .. 16f+15 form one
// contiguous 1 KB run in which 16-byte chunk l holds row 16f + (l % 16), slice bytes
// (l / 16) * 16 .. +16 -- the chunk MFMA lane l consumes.  Runs are ordered
// (matrix, fragment, slice), so a wave reads each fragment front to back in whole runs.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

__global__ __launch_bounds__(256) void pack_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                   int64_t n_chunks, int rows, int row_bytes) {
  const int nsteps = row_bytes / 64;
  const int nfrag = rows / 16;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t c = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; c < n_chunks; c += stride) {
    const int lane = static_cast<int>(c & 63);
    int64_t t = c >> 6;
    const int step = static_cast<int>(t % nsteps);
    t /= nsteps;
    const int frag = static_cast<int>(t % nfrag);
    const int64_t mat = t / nfrag;
    const int64_t row = mat * rows + frag * 16 + (lane & 15);
    const int64_t s = row * row_bytes + step * 64 + (lane >> 4) * 16;
    *reinterpret_cast<u32x4*>(dst + c * 16) = *reinterpret_cast<const u32x4*>(src + s);
  }
}

// Each wave reads its own contiguous span of span16 16-byte chunks front to back, one
// 1 KB row of the wave per load and kReadUnroll loads in flight (non-temporal), the way
// a GEMM wave walks its packed weight fragments; the workgroup leaves one XOR word in
// sink[blockIdx.x] so the loads cannot be dropped.
constexpr int kReadUnroll = 8;

__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4* __restrict__ src, int64_t n16, int64_t span16,
                                                         uint32_t* __restrict__ sink) {
  __shared__ uint32_t wx[4];
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const int64_t begin = (static_cast<int64_t>(blockIdx.x) * 4 + w) * span16;
  const int64_t end = begin + span16 < n16 ? begin + span16 : n16;
  uint32_t x = 0;
  int64_t c = begin + lane;
  for (; c + (kReadUnroll - 1) * kWave < end; c += kReadUnroll * kWave) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = __builtin_nontemporal_load(src + c + u * kWave);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; c < end; c += kWave) {
    const u32x4 v = __builtin_nontemporal_load(src + c);
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(x), o, kWave));
  if (lane == 0) wx[w] = x;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = wx[0] ^ wx[1] ^ wx[2] ^ wx[3];
}

// MFMA throughput probe: each wave runs `iters` rounds of kProbeChains independent
// accumulator chains, one MFMA per chain per round, on operands held in registers (no
// memory traffic in the loop), so the launch time measures the matrix cores' sustained
// rate at the clock the chip holds under that load.  bf16: 16x16x32 (16384 FLOP per
// MFMA); E4M3: 16x16x128 of the f8f6f4 family (65536 FLOP).  Lane 0 of each workgroup
// writes the sum of its accumulators to sink, so the work cannot be dropped.
//
// Each chain has its own B operand and the first round is peeled, so the loop carries
// eight distinct MFMA results.  With identical chains started from zero accumulators the
// compiler merges them and then rotates the 16x16 bf16 accumulators through AGPR copies
// every round (about 50 moves per 8 MFMAs), which caps the loop at about 55% of the
// matrix cores' rate; in this form the loop is 8 MFMAs and the branch.
constexpr int kProbeChains = 8;

template <int EL>
__device__ __forceinline__ f32x4 probe_mfma(const u32x4& a, const u32x4& b, f32x4 c) {
  if constexpr (EL == EL_E4M3)
    return mfma_e4m3_pair(a, b, b, a, c);
  else
    return mfma_chunk<EL_BF16>(a, b, c);
}

template <int EL>
__global__ __launch_bounds__(256) void mfma_probe_kernel(int iters, float* __restrict__ sink) {
  // small finite operands (bf16 1/128 pairs; E4M3 1.0) that differ per lane
  const uint32_t base = EL == EL_E4M3 ? 0x38383838u : 0x3C003C00u;
  const uint32_t t = threadIdx.x & 3;
  const u32x4 a = {base, base ^ (t << 8), base, base ^ t};
  u32x4 b[kProbeChains];
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c) b[c] = u32x4{base ^ t, base ^ (uint32_t)c, base ^ (t << 8), base};
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  f32x4 acc[kProbeChains];
#pragma unroll
  for (int c = 0; c < kProbeChains; ++c) acc[c] = probe_mfma<EL>(a, b[c], zero);
  for (int i = 1; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kProbeChains; ++c) acc[c] = probe_mfma<EL>(a, b[c], acc[c]);
  }
  f32x4 s = acc[0];
#pragma unroll
  for (int c = 1; c < kProbeChains; ++c) s += acc[c];
  if (threadIdx.x == 0) sink[blockIdx.x] = s[0] + s[1] + s[2] + s[3];
}

}  // namespace

hipError_t launch_mfma_probe(int el, int iters, float* sink, hipStream_t stream) {
  if (el == EL_E4M3)
    hipLaunchKernelGGL(mfma_probe_kernel<EL_E4M3>, dim3(kMfmaProbeBlocks), dim3(256), 0, stream, iters, sink);
  else
    hipLaunchKernelGGL(mfma_probe_kernel<EL_BF16>, dim3(kMfmaProbeBlocks), dim3(256), 0, stream, iters, sink);
  return hipGetLastError();
}

hipError_t launch_read_probe(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream) {
  const int64_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  // 128 KB per wave, or more so that the grid stays within kReadProbeBlocks workgroups
  const int64_t min_span = (n16 + 4ll * kReadProbeBlocks - 1) / (4ll * kReadProbeBlocks);
  const int64_t span16 = min_span > 8192 ? min_span : 8192;
  const int blocks = static_cast<int>((n16 + 4 * span16 - 1) / (4 * span16));
  hipLaunchKernelGGL(read_probe_kernel, dim3(blocks), dim3(256), 0, stream, static_cast<const u32x4*>(src), n16,
                     span16, sink);
  return hipGetLastError();
}

hipError_t launch_pack(const void* src, void* dst, int64_t n_mats, int rows, int row_bytes, hipStream_t stream) {
  const int64_t n_chunks = n_mats * rows * (row_bytes / 16);
  if (n_chunks == 0) return hipSuccess;
  const int64_t want = (n_chunks + 255) / 256;
  const int blocks = static_cast<int>(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(pack_kernel, dim3(blocks), dim3(256), 0, stream, static_cast<const uint8_t*>(src),
                     static_cast<uint8_t*>(dst), n_chunks, rows, row_bytes);
  return hipGetLastError();
}

}  // namespace moe
