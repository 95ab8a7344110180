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

}  // namespace

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
