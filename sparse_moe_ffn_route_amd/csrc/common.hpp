// Device helpers shared by the gfx950 kernels of the MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Element types of GEMM operands and outputs (same values as enum moe_dtype).
enum : int { EL_F32 = 0, EL_BF16 = 1, EL_E4M3 = 2 };

template <int EL> struct ElSize;
template <> struct ElSize<EL_F32> { static constexpr int v = 4; };
template <> struct ElSize<EL_BF16> { static constexpr int v = 2; };
template <> struct ElSize<EL_E4M3> { static constexpr int v = 1; };

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Scalar conversions
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Two floats -> two OCP E4M3 codes in the low 16 bits (hardware convert, nearest even).
// Callers clamp to +-448 first, so the convert never sees an out-of-range value.
__device__ __forceinline__ uint32_t f32x2_to_e4m3x2(float a, float b) {
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false)) & 0xFFFFu;
}

// Raw buffer access: a wave-uniform 128-bit resource (base address, no stride, no range
// limit in practice) plus a 32-bit per-lane offset and a 32-bit wave-uniform offset.
// Loads through it need no per-lane 64-bit address arithmetic, so a loop can advance a
// stream by changing only the uniform offset.  Word 3 is the gfx9-family default format
// (32-bit data, no swizzle).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base) {
  // readfirstlane returns int: each half goes back through uint32_t before widening, so
  // an address with bit 31 set is not sign-extended into the upper half
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a)));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32)));
  const uint64_t u = (static_cast<uint64_t>(hi) << 32) | lo;
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(u), 0, -1, 0x00020000);
}

// A resource with no records: every load through it is out of range, returns zeros and
// touches no memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc_empty() {
  return __builtin_amdgcn_make_buffer_rsrc(nullptr, 0, 0, 0x00020000);
}

// NT: non-temporal hint (stream the lines through the caches without keeping them).
template <bool NT = false>
__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, NT ? 2 : 0));
}

// Direct buffer-to-LDS load: every lane reads 16 bytes at the resource's base + voff +
// soff and they land in LDS at lds_wave_base + 16 * lane (one contiguous 1 KB per wave;
// lds_wave_base must be wave-uniform).  Counted by vmcnt like any vector load.
__device__ __forceinline__ void buffer_load16_to_lds(__amdgpu_buffer_rsrc_t r, void* lds_wave_base, uint32_t voff,
                                                     uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_wave_base, 16, voff, soff,
                                           0, 0);
}

// Wait until at most N vector memory operations of this wave are outstanding (N <= 63).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier without a memory fence (the compiler's fence would wait for every
// vector load in flight while LDS-bound loads are outstanding); memory operations are
// kept on their side of it.  Callers make their own LDS writes complete first.
__device__ __forceinline__ void bare_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Two floats -> two bfloat16 (low half = a), round to nearest even; one gfx950 convert.
__device__ __forceinline__ uint32_t bf16x2_bits(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

// silu(z) = z * sigmoid(z) = z / (1 + e^-z), with the hardware reciprocal (about 1 ulp):
// for z -> -inf the reciprocal of +inf is 0 and the result is -0, for z -> +inf it is z.
__device__ __forceinline__ float silu(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// ---------------------------------------------------------------------------
// One 16-byte K-chunk per lane through the 16x16 MFMA family.
//
// A wave holds a 16-row A tile and a 16-column B tile, each lane carrying 16
// contiguous bytes of its row (A) / column (B) at K-offset (lane / 16) * 16 bytes.
// The four lane groups therefore cover 64 contiguous bytes of K; the element
// order inside the MFMA is the same for A and B, so the dot products are the
// plain K-sums.  The accumulator layout is the 16x16 MFMA one: lane l holds
// C[(l / 16) * 4 + r][l % 16], r = 0..3 (row of A, column of B).
// ---------------------------------------------------------------------------

template <int EL> __device__ __forceinline__ f32x4 mfma_chunk(const u32x4& a, const u32x4& b, f32x4 c);

template <> __device__ __forceinline__ f32x4 mfma_chunk<EL_BF16>(const u32x4& a, const u32x4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                 c, 0, 0, 0);
}

template <> __device__ __forceinline__ f32x4 mfma_chunk<EL_F32>(const u32x4& a, const u32x4& b, f32x4 c) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
  return c;
}

template <> __device__ __forceinline__ f32x4 mfma_chunk<EL_E4M3>(const u32x4& a, const u32x4& b, f32x4 c) {
  long a0 = static_cast<long>((static_cast<uint64_t>(a.y) << 32) | a.x);
  long a1 = static_cast<long>((static_cast<uint64_t>(a.w) << 32) | a.z);
  long b0 = static_cast<long>((static_cast<uint64_t>(b.y) << 32) | b.x);
  long b1 = static_cast<long>((static_cast<uint64_t>(b.w) << 32) | b.z);
  c = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a0, b0, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a1, b1, c, 0, 0, 0);
  return c;
}

// Two 16-byte E4M3 K-chunks per lane (the chunks of two consecutive 64-byte K slices,
// A and B alike) through one 16x16x128 MFMA of gfx950's f8f6f4 family: both operands
// OCP E4M3 (format code 0), block scales 2^0 (E8M0 127).  Which K index each byte
// stands for does not matter as long as A and B use the same arrangement, which they do.
typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mfma_e4m3_pair(const u32x4& a0, const u32x4& a1, const u32x4& b0, const u32x4& b1,
                                                f32x4 c) {
  const i32x8 a = __builtin_bit_cast(i32x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
  const i32x8 b = __builtin_bit_cast(i32x8, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7));
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// ---------------------------------------------------------------------------
// Wave helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Wave-uniform read of a value no thread writes during the kernel (e.g. a prefix
// array written by an earlier launch), through the scalar data cache: it is counted
// apart from the vector loads, so waiting for it never waits for a pending weight
// stream.  Reads only.
template <typename T>
__device__ __forceinline__ T ld_scalar(const T* p) {
  return *(const __attribute__((address_space(4))) T*)(p);
}

// Map a linear block index onto a contiguous range of logical tiles per XCD.
// Blocks are dispatched round-robin over the 8 XCDs of an MI355X, so block b runs on
// XCD b % 8; giving each XCD one contiguous range keeps tiles that share operands
// (the same expert's weights, the same token rows) in one L2.
__device__ __forceinline__ int xcd_remap(int b, int total) {
  const int q = total / 8, r = total % 8;
  const int xcd = b % 8, local = b / 8;
  return xcd * q + (xcd < r ? xcd : r) + local;
}

}  // namespace moe
