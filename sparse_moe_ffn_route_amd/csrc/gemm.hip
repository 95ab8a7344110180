// Ragged grouped GEMM of the expert FFNs (and the router projection), gfx950 MFMA.
//
// Source: the "Grouped GEMMs" block of "Systems Engineering Playbook: Qwen 3.5 MoE on
// Ironwood TPU" (introduction and table "Three High-Leverage Optimizations"); the
// SwiGLU form of the experts is this library's reading of "3. Sparse
// Mixture-of-Experts (MoE)" in "Tối ưu hóa mô hình Qwen 3.5-397B MoE trên hạ tầng TPU
// Ironwood", whose formula is missing.
//
// Work unit (one 256-thread workgroup): one (group, M-tile, N-tile).  The M-tile is
// 16 or 32 rows of the group (token rows, gathered through perm), the N-tile is
// 4 waves x NF x 16 output channels (for SwiGLU the same channels of W_gate and
// W_up, so silu(gate) * up is formed in registers).
//
// Data path, chosen for the weight-streaming regime where each expert has few rows:
//   * weights go straight from HBM into VGPRs as the MFMA "A" operand: lane l of a
//     wave reads 16 bytes of output channel (l % 16) at K-byte offset (l / 16) * 16,
//     so a wave reads 16 rows x 64 contiguous bytes per K step; a K block is 8 steps
//     (512 bytes of every row), double-buffered in registers (ping-pong), so one
//     block's loads are in flight while the previous block is multiplied;
//   * token rows are the MFMA "B" operand, staged per K block in LDS (double
//     buffered, one barrier per block) because every wave of the workgroup uses them;
//   * each weight byte is read once per M-tile; M-tiles of one expert are neighbours
//     in the tile order so repeats hit L2.
// Tiles are ordered (group, M-tile, N-tile) and dealt to XCDs in contiguous ranges.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kKSteps = 8;                // 64-byte K steps per K block
constexpr int kKBlk = kKSteps * 64;       // bytes of each row per K block
constexpr int kLdsRow = kKBlk + 16;       // padded LDS row (bytes)

template <int OUT> struct OutStore;

template <> struct OutStore<EL_F32> {
  static __device__ __forceinline__ void store4(void* base, size_t idx, const float v[4], int valid) {
    float* p = static_cast<float*>(base) + idx;
    if (valid >= 4 && (idx & 3) == 0) {
      *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    } else {
      for (int r = 0; r < (valid < 4 ? valid : 4); ++r) p[r] = v[r];
    }
  }
};

template <> struct OutStore<EL_BF16> {
  static __device__ __forceinline__ void store4(void* base, size_t idx, const float v[4], int valid) {
    uint16_t* p = static_cast<uint16_t*>(base) + idx;
    const uint32_t b0 = f32_to_bf16_bits(v[0]), b1 = f32_to_bf16_bits(v[1]);
    const uint32_t b2 = f32_to_bf16_bits(v[2]), b3 = f32_to_bf16_bits(v[3]);
    if (valid >= 4 && (idx & 3) == 0) {
      *reinterpret_cast<uint2*>(p) = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
    } else {
      const uint32_t b[4] = {b0, b1, b2, b3};
      for (int r = 0; r < (valid < 4 ? valid : 4); ++r) p[r] = static_cast<uint16_t>(b[r]);
    }
  }
};

template <int EL, int OUT, int MF, int NF, bool SWIGLU>
__global__ __launch_bounds__(256, 2) void gemm_kernel(GemmProblem p0, GemmProblem p1, int has_p1) {
  constexpr int ES = ElSize<EL>::v;
  constexpr int BM = 16 * MF;
  constexpr int NMAT = SWIGLU ? 2 : 1;
  constexpr int BN = 4 * NF * 16;
  constexpr int CPT = BM * (kKBlk / 16) / 256;  // 16-byte A chunks per thread per K block
  __shared__ __attribute__((aligned(16))) uint8_t sA[2][BM * kLdsRow];

  // ---- which tile ---------------------------------------------------------
  const int nt0 = (p0.N + BN - 1) / BN;
  const int nt1 = has_p1 ? (p1.N + BN - 1) / BN : 1;
  const int tiles0 = (p0.offsets ? p0.tile_prefix[p0.n_groups] : (p0.rows + BM - 1) / BM) * nt0;
  const int tiles1 = has_p1 ? ((p1.rows + BM - 1) / BM) * nt1 : 0;
  const int total = tiles0 + tiles1;
  if (static_cast<int>(blockIdx.x) >= total) return;
  int L = xcd_remap(blockIdx.x, total);
  const bool sec = L >= tiles0;
  if (sec) L -= tiles0;
#define SEL(f) (sec ? p1.f : p0.f)
  const int n_tiles = sec ? nt1 : nt0;
  const int32_t* offsets = SEL(offsets);
  const int n_tile = L % n_tiles;
  const int q = L / n_tiles;
  int g = 0, m = q, row0 = 0, count = SEL(rows);
  if (offsets) {
    const int32_t* pre = SEL(tile_prefix);
    int lo = 0, hi = SEL(n_groups) - 1;
    while (lo < hi) {  // largest g with pre[g] <= q
      const int mid = (lo + hi + 1) >> 1;
      if (pre[mid] <= q) lo = mid; else hi = mid - 1;
    }
    g = lo;
    m = q - pre[g];
    row0 = offsets[g];
    count = offsets[g + 1] - row0;
  }
  const int rbeg = m * BM;
  const int nrows = min(BM, count - rbeg);
  const int N = SEL(N);
  const int Kb = SEL(K) * ES;  // bytes per row
  const uint8_t* A = static_cast<const uint8_t*>(SEL(a));
  const int32_t* perm = SEL(perm);
  const size_t lda_b = static_cast<size_t>(SEL(lda)) * ES;
  const size_t wgrp = static_cast<size_t>(g) * SEL(w_stride) * ES;
  const uint8_t* W0 = static_cast<const uint8_t*>(SEL(w0)) + wgrp;
  const uint8_t* W1 = SWIGLU ? static_cast<const uint8_t*>(SEL(w1)) + wgrp : nullptr;

  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int lrow = lane & 15, lgrp = lane >> 4;
  const int ncol0 = n_tile * BN + wave * NF * 16;

  // ---- operand pointers ---------------------------------------------------
  const uint8_t* wrow[NMAT][NF];
#pragma unroll
  for (int nf = 0; nf < NF; ++nf) {
    const int n = min(ncol0 + nf * 16 + lrow, N - 1);
    wrow[0][nf] = W0 + static_cast<size_t>(n) * Kb + lgrp * 16;
    if (SWIGLU) wrow[NMAT - 1][nf] = W1 + static_cast<size_t>(n) * Kb + lgrp * 16;
  }
  const uint8_t* arow[CPT];
  int acol[CPT], aoff[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = threadIdx.x + i * 256;
    const int r = c / (kKBlk / 16);
    acol[i] = (c % (kKBlk / 16)) * 16;
    aoff[i] = r * kLdsRow + acol[i];
    arow[i] = nullptr;
    if (r < nrows) {
      const int grow = row0 + rbeg + r;
      const int src = perm ? perm[grow] : grow;
      arow[i] = A + static_cast<size_t>(src) * lda_b;
    }
  }

  f32x4 acc[NMAT][NF][MF];
#pragma unroll
  for (int a = 0; a < NMAT; ++a)
#pragma unroll
    for (int nf = 0; nf < NF; ++nf)
#pragma unroll
      for (int mf = 0; mf < MF; ++mf) acc[a][nf][mf] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nblk = (Kb + kKBlk - 1) / kKBlk;

  auto load_w = [&](uint4 (&w)[NMAT][NF][kKSteps], int kb) {
    const int off = kb * kKBlk;
    const int steps = min(kKSteps, (Kb - off) / 64);
#pragma unroll
    for (int s = 0; s < kKSteps; ++s)
#pragma unroll
      for (int a = 0; a < NMAT; ++a)
#pragma unroll
        for (int nf = 0; nf < NF; ++nf)
          if (s < steps) w[a][nf][s] = *reinterpret_cast<const uint4*>(wrow[a][nf] + off + s * 64);
  };
  auto load_a = [&](uint4 (&av)[CPT], int kb) {
    const int off = kb * kKBlk;
    const int bytes = min(kKBlk, Kb - off);
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      av[i] = make_uint4(0, 0, 0, 0);
      if (arow[i] && acol[i] < bytes) av[i] = *reinterpret_cast<const uint4*>(arow[i] + off + acol[i]);
    }
  };
  auto store_a = [&](const uint4 (&av)[CPT], int buf) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) *reinterpret_cast<uint4*>(&sA[buf][aoff[i]]) = av[i];
  };
  auto compute = [&](const uint4 (&w)[NMAT][NF][kKSteps], int kb) {
    const int buf = kb & 1;
    const int steps = min(kKSteps, (Kb - kb * kKBlk) / 64);
#pragma unroll
    for (int s = 0; s < kKSteps; ++s) {
      if (s < steps) {
        uint4 bfr[MF];
#pragma unroll
        for (int mf = 0; mf < MF; ++mf)
          bfr[mf] = *reinterpret_cast<const uint4*>(&sA[buf][(mf * 16 + lrow) * kLdsRow + s * 64 + lgrp * 16]);
#pragma unroll
        for (int a = 0; a < NMAT; ++a)
#pragma unroll
          for (int nf = 0; nf < NF; ++nf)
#pragma unroll
            for (int mf = 0; mf < MF; ++mf) acc[a][nf][mf] = mfma_chunk<EL>(w[a][nf][s], bfr[mf], acc[a][nf][mf]);
      }
    }
  };

  // ---- main loop: ping-pong register buffers for the weights ---------------
  uint4 wA[NMAT][NF][kKSteps], wB[NMAT][NF][kKSteps];
  uint4 av[CPT];
  load_w(wA, 0);
  load_a(av, 0);
  store_a(av, 0);
  __syncthreads();
  for (int kb = 0; kb < nblk; kb += 2) {
    if (kb + 1 < nblk) {
      load_w(wB, kb + 1);
      load_a(av, kb + 1);
    }
    compute(wA, kb);
    if (kb + 1 < nblk) store_a(av, (kb + 1) & 1);
    __syncthreads();
    if (kb + 1 >= nblk) break;
    if (kb + 2 < nblk) {
      load_w(wA, kb + 2);
      load_a(av, kb + 2);
    }
    compute(wB, kb + 1);
    if (kb + 2 < nblk) store_a(av, (kb + 2) & 1);
    __syncthreads();
  }

  // ---- epilogue -------------------------------------------------------------
  void* out = SEL(out);
  const size_t ldo = SEL(ldo);
  const float* a_scale = SEL(a_scale);
  const float* s0 = SEL(s0);
  const float* s1 = SEL(s1);
#pragma unroll
  for (int mf = 0; mf < MF; ++mf) {
    const int r = mf * 16 + lrow;
    if (r >= nrows) continue;
    const int grow = row0 + rbeg + r;
    float as = 1.0f;
    if (EL == EL_E4M3) as = a_scale[perm ? perm[grow] : grow];
#pragma unroll
    for (int nf = 0; nf < NF; ++nf) {
      const int n = ncol0 + nf * 16 + lgrp * 4;
      if (n >= N) continue;
      const int valid = min(4, N - n);
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x0 = acc[0][nf][mf][i];
        if (EL == EL_E4M3) x0 *= as * s0[static_cast<size_t>(g) * N + min(n + i, N - 1)];
        if (SWIGLU) {
          float x1 = acc[NMAT - 1][nf][mf][i];
          if (EL == EL_E4M3) x1 *= as * s1[static_cast<size_t>(g) * N + min(n + i, N - 1)];
          v[i] = silu(x0) * x1;
        } else {
          v[i] = x0;
        }
      }
      OutStore<OUT>::store4(out, static_cast<size_t>(grow) * ldo + n, v, valid);
    }
  }
#undef SEL
}

template <int EL, int OUT, int MF, int NF, bool SWIGLU>
hipError_t launch_one(const GemmProblem& p0, const GemmProblem* p1, int max_tiles0, hipStream_t stream) {
  constexpr int BM = 16 * MF, BN = 4 * NF * 16;
  int tiles1 = 0;
  GemmProblem q1 = p0;
  if (p1) {
    q1 = *p1;
    tiles1 = ((p1->rows + BM - 1) / BM) * ((p1->N + BN - 1) / BN);
  }
  const int grid = max_tiles0 + tiles1;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_kernel<EL, OUT, MF, NF, SWIGLU>), dim3(grid), dim3(256), 0, stream, p0, q1,
                     p1 ? 1 : 0);
  return hipGetLastError();
}

template <int EL, int OUT, bool SWIGLU>
hipError_t launch_mf(int mf, const GemmProblem& p0, const GemmProblem* p1, int max_tiles0, hipStream_t stream) {
  constexpr int NF = SWIGLU ? 1 : 2;
  if (mf == 1) return launch_one<EL, OUT, 1, NF, SWIGLU>(p0, p1, max_tiles0, stream);
  return launch_one<EL, OUT, 2, NF, SWIGLU>(p0, p1, max_tiles0, stream);
}

}  // namespace

int gemm_bm(int mf) { return 16 * mf; }

int gemm_bn(bool swiglu) { return 4 * (swiglu ? 1 : 2) * 16; }

hipError_t launch_gemm(int el, int out_el, bool swiglu, int mf, const GemmProblem& p0, const GemmProblem* p1,
                       int max_tiles0, hipStream_t stream) {
  if (swiglu) {
    if (el == EL_F32 && out_el == EL_F32) return launch_mf<EL_F32, EL_F32, true>(mf, p0, p1, max_tiles0, stream);
    if (el == EL_BF16 && out_el == EL_BF16) return launch_mf<EL_BF16, EL_BF16, true>(mf, p0, p1, max_tiles0, stream);
    if (el == EL_E4M3 && out_el == EL_BF16) return launch_mf<EL_E4M3, EL_BF16, true>(mf, p0, p1, max_tiles0, stream);
  } else {
    if (el == EL_F32 && out_el == EL_F32) return launch_mf<EL_F32, EL_F32, false>(mf, p0, p1, max_tiles0, stream);
    if (el == EL_BF16 && out_el == EL_BF16) return launch_mf<EL_BF16, EL_BF16, false>(mf, p0, p1, max_tiles0, stream);
    if (el == EL_BF16 && out_el == EL_F32) return launch_mf<EL_BF16, EL_F32, false>(mf, p0, p1, max_tiles0, stream);
    if (el == EL_E4M3 && out_el == EL_BF16) return launch_mf<EL_E4M3, EL_BF16, false>(mf, p0, p1, max_tiles0, stream);
    if (el == EL_E4M3 && out_el == EL_F32) return launch_mf<EL_E4M3, EL_F32, false>(mf, p0, p1, max_tiles0, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
