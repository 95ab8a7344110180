// Ragged grouped GEMM of the expert FFNs (and the router projection), gfx950 MFMA.
//
// Source: the "Grouped GEMMs" block of "Systems Engineering Playbook: Qwen 3.5 MoE on
// Ironwood TPU" (introduction and table "Three High-Leverage Optimizations"); the
// SwiGLU form of the experts is this library's reading of "3. Sparse
// Mixture-of-Experts (MoE)" in "Tối ưu hóa mô hình Qwen 3.5-397B MoE trên hạ tầng TPU
// Ironwood", whose formula is missing.
//
// Work unit (one 256-thread workgroup): one (group, N-tile, M-tile).  The M-tile is up
// to 16 * MF token rows of the group (gathered through perm); the N-tile is
// 4 waves x NF x 16 output channels (for SwiGLU the same channels of W_gate and W_up,
// so silu(gate) * up is formed in registers).
//
// Data path:
//   * weights go straight from HBM into VGPRs as the MFMA "A" operand; each wave owns
//     its own output channels, so weights are never shared between waves and need no
//     LDS.  Lane l of a wave reads 16 bytes of channel (l % 16) at K-byte offset
//     (l / 16) * 16, so one wave step covers 16 rows x 64 contiguous bytes; K blocks
//     of KSTEPS steps rotate through a ring of NBUF register buffers, so the loads of
//     the next NBUF - 1 blocks are in flight while one block is multiplied;
//   * token rows are the MFMA "B" operand, shared by the 4 waves: staged per K block in
//     LDS (double-buffered, one barrier per block), loaded before the weights of the
//     same block so the LDS store never waits for the weight stream;
//   * 16-row token fragments past the tile's last row are skipped (uniform branch), so
//     a ragged group costs MFMA time in 16-row steps only.
// Two shapes are instantiated: a streaming shape (MF = 1 or 2, two buffers, two
// workgroups per CU; the down projection takes 4 fragments per wave to double the
// channels each workgroup streams) for the few-rows-per-expert decode regime, where
// each weight byte feeds one tile and the kernel is an HBM stream; and a tile shape
// (MF = 16, 2-step blocks, three buffers, 2 fragments per matrix per wave, one
// workgroup per CU so a wave may hold 512 registers) for the prefill regime: a 256-row
// M-tile covers every row of a typical expert (~160 at 8K tokens), so each weight byte
// is streamed from HBM once and feeds all of the expert's rows, and 32 channels per
// matrix per wave halve the token bytes staged per MFMA; only experts with more rows
// (skewed routing) take several M-tiles, adjacent in the launch order.
// Tiles are ordered (group, N-tile, M-tile) and dealt to XCDs in contiguous ranges.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

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
    const uint32_t b01 = bf16x2_bits(v[0], v[1]), b23 = bf16x2_bits(v[2], v[3]);
    if (valid >= 4 && (idx & 3) == 0) {
      *reinterpret_cast<uint2*>(p) = make_uint2(b01, b23);
    } else {
      const uint32_t b[4] = {b01 & 0xFFFFu, b01 >> 16, b23 & 0xFFFFu, b23 >> 16};
      for (int r = 0; r < (valid < 4 ? valid : 4); ++r) p[r] = static_cast<uint16_t>(b[r]);
    }
  }
};

constexpr int gcd_c(int a, int b) { return b == 0 ? a : gcd_c(b, a % b); }

template <bool NT>
__device__ __forceinline__ u32x4 load_weight(const uint8_t* p) {
  if (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return *reinterpret_cast<const u32x4*>(p);
}

template <int EL, int OUT, int MF, int NF, bool SWIGLU, int KSTEPS, int NBUF, bool NTW, int MINB, bool PACKED,
          int TDEPTH>
__global__ __launch_bounds__(256, MINB) void gemm_kernel(GemmProblem p0, GemmProblem p1, int has_p1) {
  constexpr int ES = ElSize<EL>::v;
  constexpr int BM = 16 * MF;
  constexpr int NMAT = SWIGLU ? 2 : 1;
  constexpr int BN = 4 * NF * 16;
  constexpr int KBLK = KSTEPS * 64;   // bytes of each row per K block
  constexpr int LDS_ROW = KBLK + 16;  // padded LDS row (bytes)
  constexpr int CHUNKS = BM * (KBLK / 16);
  static_assert(CHUNKS % 256 == 0, "token tile must split evenly over 256 threads");
  constexpr int CPT = CHUNKS / 256;   // 16-byte token chunks per thread per K block
  __shared__ __attribute__((aligned(16))) uint8_t sA[2][BM * LDS_ROW];

  // ---- which tile ---------------------------------------------------------
  const int nt0 = (p0.N + BN - 1) / BN;
  const int nt1 = has_p1 ? (p1.N + BN - 1) / BN : 1;
  const int tiles0 = (p0.offsets ? p0.tile_prefix[p0.n_groups] : (p0.rows + BM - 1) / BM * p0.k_splits) * nt0;
  const int tiles1 = has_p1 ? ((p1.rows + BM - 1) / BM) * p1.k_splits * nt1 : 0;
  const int total = tiles0 + tiles1;
  if (static_cast<int>(blockIdx.x) >= total) return;
  int L = xcd_remap(blockIdx.x, total);
  const bool sec = L >= tiles0;
  if (sec) L -= tiles0;
#define SEL(f) (sec ? p1.f : p0.f)
  const int n_tiles = sec ? nt1 : nt0;
  const int32_t* offsets = SEL(offsets);
  int g = 0, row0 = 0, count = SEL(rows), n_tile, m, ks = 0;
  const int ksp = SEL(k_splits);
  if (offsets) {
    // group g owns tiles [pre[g] * n_tiles, pre[g + 1] * n_tiles), ordered (N-tile, M-tile)
    const int32_t* pre = SEL(tile_prefix);
    const int q = L / n_tiles;
    int lo = 0, hi = SEL(n_groups) - 1;
    while (lo < hi) {  // largest g with pre[g] <= q
      const int mid = (lo + hi + 1) >> 1;
      if (pre[mid] <= q) lo = mid; else hi = mid - 1;
    }
    g = lo;
    const int mt = pre[g + 1] - pre[g];
    const int local = L - pre[g] * n_tiles;
    n_tile = local / mt;
    m = local % mt;
    row0 = offsets[g];
    count = offsets[g + 1] - row0;
  } else {
    const int mt = (count + BM - 1) / BM;
    m = L % mt;
    ks = (L / mt) % ksp;
    n_tile = L / mt / ksp;
  }
  // the tile coordinates are wave-uniform; say so, so that addresses built from them
  // stay in scalar registers
  g = __builtin_amdgcn_readfirstlane(g);
  row0 = __builtin_amdgcn_readfirstlane(row0);
  count = __builtin_amdgcn_readfirstlane(count);
  n_tile = __builtin_amdgcn_readfirstlane(n_tile);
  m = __builtin_amdgcn_readfirstlane(m);
  ks = __builtin_amdgcn_readfirstlane(ks);
  const int rbeg = m * BM;
  const int nrows = min(BM, count - rbeg);
  const int N = SEL(N);
  const int Kb_row = SEL(K) * ES;  // bytes per row
  const int Kb = Kb_row / ksp;     // bytes of this K range
  const int kofs = ks * Kb;
  const uint8_t* A = static_cast<const uint8_t*>(SEL(a)) + kofs;
  const int32_t* perm = SEL(perm);
  const size_t lda_b = static_cast<size_t>(SEL(lda)) * ES;
  const size_t wgrp = static_cast<size_t>(g) * SEL(w_stride) * ES;
  const uint8_t* W0 = static_cast<const uint8_t*>(SEL(w0)) + wgrp;
  const uint8_t* W1 = SWIGLU ? static_cast<const uint8_t*>(SEL(w1)) + wgrp : nullptr;
  // Weight addressing: row-major rows are Kb_row apart and a 64-byte step is 64 bytes on;
  // in the packed layout a 16-row fragment is one run of 1 KB per step.
  constexpr int SSTEP = PACKED ? 1024 : 64;     // bytes between consecutive 64-byte K steps
  constexpr int SBLK = KSTEPS * SSTEP;          // bytes between consecutive K blocks

  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int lrow = lane & 15, lgrp = lane >> 4;
  const int ncol0 = n_tile * BN + wave * NF * 16;
  const int mf_active = (nrows + 15) / 16;

  // Full K blocks run a branch-free pipeline; a last partial block (K*ES not a
  // multiple of KBLK) is handled after it with per-step guards.
  const int nfull = Kb / KBLK;
  const int tail_steps = (Kb - nfull * KBLK) / 64;

  // ---- epilogue: scales, SwiGLU, store --------------------------------------
  auto epilogue = [&](const f32x4 (&acc)[NMAT][NF][MF]) {
    void* out = static_cast<uint8_t*>(SEL(out)) + static_cast<size_t>(ks) * SEL(out_split_stride) * (OUT == EL_F32 ? 4 : 2);
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
  };

  if constexpr (MF >= 8) {
    // ---- tile shape ---------------------------------------------------------
    // Weights and token rows are read through buffer resources: a wave-uniform base, a
    // fixed 32-bit offset per lane, and the K-block offset as the uniform part, so the
    // loop computes no per-lane addresses (the host keeps every offset below 2^31).
    // Token rows past the tile's last row re-read its last row (harmless: those output
    // rows are never stored), so every load in the loop is unconditional.  The K loop
    // is specialised on the number of 16-row fragments actually in use (rounded up to a
    // multiple of kFragGroup), so the fragment loop has no branches and the LDS reads
    // run one fragment ahead of the MFMAs.
    constexpr int kFragGroup = 2;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int ncol0u = n_tile * BN + wv * NF * 16;
    __amdgpu_buffer_rsrc_t wres[NMAT];
    wres[0] = buffer_rsrc(W0);
    if (SWIGLU) wres[NMAT - 1] = buffer_rsrc(W1);
    uint32_t woff_v[NF], woff_s[NF];
#pragma unroll
    for (int nf = 0; nf < NF; ++nf) {
      if (PACKED) {
        const int frag = min((ncol0u + nf * 16) / 16, N / 16 - 1);
        woff_s[nf] = (static_cast<uint32_t>(frag) * (Kb_row / 64) + kofs / 64) * 1024;
        woff_v[nf] = lane * 16;
      } else {
        const int n = min(ncol0u + nf * 16 + lrow, N - 1);
        woff_s[nf] = kofs;
        woff_v[nf] = static_cast<uint32_t>(n) * Kb_row + lgrp * 16;
      }
    }
    constexpr int CPR = KBLK / 16;        // 16-byte chunks per token row per K block
    constexpr int RPP = 256 / CPR;        // token rows per pass of the workgroup
    constexpr int NTP = BM / RPP;         // passes for a full tile
    const int crow = threadIdx.x / CPR, ccol = (threadIdx.x % CPR) * 16;
    const __amdgpu_buffer_rsrc_t tres = buffer_rsrc(A);
    uint32_t toff[NTP];
#pragma unroll
    for (int i = 0; i < NTP; ++i) {
      const int grow = row0 + rbeg + min(crow + i * RPP, nrows - 1);
      toff[i] = static_cast<uint32_t>(perm ? perm[grow] : grow) * static_cast<uint32_t>(lda_b) + ccol;
    }
    const int tl_off = crow * LDS_ROW + ccol;
    const int b_off = lrow * LDS_ROW + lgrp * 16;

    auto run = [&](auto mfr_c) {
      constexpr int MFR = decltype(mfr_c)::value;      // fragments computed
      constexpr int NTL = (MFR * 16 + RPP - 1) / RPP;  // token passes they need
      f32x4 acc[NMAT][NF][MF];
#pragma unroll
      for (int a = 0; a < NMAT; ++a)
#pragma unroll
        for (int nf = 0; nf < NF; ++nf)
#pragma unroll
          for (int mf = 0; mf < MF; ++mf) acc[a][nf][mf] = f32x4{0.f, 0.f, 0.f, 0.f};
      u32x4 wr[NBUF][NMAT][NF][KSTEPS];
      u32x4 tv[TDEPTH][NTL];  // token rows of the next TDEPTH blocks, in flight
      auto ld_w = [&](u32x4 (&w)[NMAT][NF][KSTEPS], int kb) {
        const uint32_t o = static_cast<uint32_t>(min(kb, nfull - 1)) * SBLK;
#pragma unroll
        for (int st = 0; st < KSTEPS; ++st)
#pragma unroll
          for (int a = 0; a < NMAT; ++a)
#pragma unroll
            for (int nf = 0; nf < NF; ++nf)
              w[a][nf][st] = buffer_load16<NTW>(wres[a], woff_v[nf], woff_s[nf] + o + st * SSTEP);
      };
      auto ld_t = [&](u32x4 (&t)[NTL], int kb) {
        const uint32_t o = static_cast<uint32_t>(min(kb, nfull - 1)) * KBLK;
#pragma unroll
        for (int i = 0; i < NTL; ++i) t[i] = buffer_load16(tres, toff[i], o);
      };
      auto st_t = [&](const u32x4 (&t)[NTL], int buf) {
#pragma unroll
        for (int i = 0; i < NTL; ++i) *reinterpret_cast<u32x4*>(&sA[buf][tl_off + i * RPP * LDS_ROW]) = t[i];
      };
      // Token fragments are read kLdsAhead fragments ahead of the MFMAs that use them
      // (a ring of kLdsAhead + 1 registers); the scheduling barriers keep that order
      // (the scheduler would otherwise hoist every read of the block and run out of
      // registers).
      constexpr int kLdsAhead = 1;
      constexpr int NQ = kLdsAhead + 1;
      auto mm = [&](const u32x4 (&w)[NMAT][NF][KSTEPS], int buf, int nst) {
        const uint8_t* sb = &sA[buf][b_off];
        const int total = nst * MFR;  // (step, fragment) pairs of this block, in issue order
        auto frag_at = [&](int q) {
          return *reinterpret_cast<const u32x4*>(sb + (q % MFR) * 16 * LDS_ROW + (q / MFR) * 64);
        };
        if constexpr (EL == EL_E4M3 && KSTEPS % 2 == 0) {
          // E4M3: K slices in pairs through the 16x16x128 MFMA, one fragment's pair ahead;
          // a lone last slice (odd tail) is paired with zeros on both sides.
          constexpr int NP = KSTEPS / 2;
          const int npairs = (nst + 1) / 2;
          const u32x4 z = {0u, 0u, 0u, 0u};
          u32x4 bl[2], bh[2];
          auto rd = [&](int q, u32x4& lo, u32x4& hi) {
            const int sp = q / MFR, mf = q % MFR;
            lo = frag_at((2 * sp) * MFR + mf);
            hi = 2 * sp + 1 < nst ? frag_at((2 * sp + 1) * MFR + mf) : z;
          };
          rd(0, bl[0], bh[0]);
#pragma unroll
          for (int sp = 0; sp < NP; ++sp) {
            if (sp >= npairs) break;
            const bool two = 2 * sp + 1 < nst;
#pragma unroll
            for (int mf = 0; mf < MFR; ++mf) {
              const int cur = sp * MFR + mf, nx = cur + 1;
              if (nx < NP * MFR && nx / MFR < npairs) rd(nx, bl[nx & 1], bh[nx & 1]);
#pragma unroll
              for (int a = 0; a < NMAT; ++a)
#pragma unroll
                for (int nf = 0; nf < NF; ++nf)
                  acc[a][nf][mf] = mfma_e4m3_pair(w[a][nf][2 * sp], two ? w[a][nf][2 * sp + 1] : z, bl[cur & 1],
                                                  bh[cur & 1], acc[a][nf][mf]);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
          return;
        }
        u32x4 bq[NQ];
#pragma unroll
        for (int q = 0; q < kLdsAhead; ++q)
          if (q < KSTEPS * MFR && q < total) bq[q] = frag_at(q);
#pragma unroll
        for (int st = 0; st < KSTEPS; ++st) {
          if (st >= nst) break;
#pragma unroll
          for (int mf = 0; mf < MFR; ++mf) {
            const int cur = st * MFR + mf;
            const int nx = cur + kLdsAhead;
            if (nx < KSTEPS * MFR && nx < total) bq[nx % NQ] = frag_at(nx);
#pragma unroll
            for (int a = 0; a < NMAT; ++a)
#pragma unroll
              for (int nf = 0; nf < NF; ++nf)
                acc[a][nf][mf] = mfma_chunk<EL>(w[a][nf][st], bq[cur % NQ], acc[a][nf][mf]);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      };
      // Block b's token rows are loaded TDEPTH blocks ahead into tv[b % TDEPTH] and
      // stored to LDS buffer b & 1 at the end of block b - 1; its weights are loaded
      // NBUF - 1 blocks ahead into wr[b % NBUF].  The loop is unrolled over
      // lcm(NBUF, TDEPTH) blocks so both ring indices are compile-time constants.
      // Loads complete in issue order, so waiting for a block's token rows also waits
      // for every older load: with TDEPTH = NBUF - 1 the token rows of block b + 1 are
      // issued together with its weights, and that wait never holds up a weight
      // prefetch that is still needed later.
      constexpr int U = NBUF * TDEPTH / gcd_c(NBUF, TDEPTH);
      if (nfull > 0) {
#pragma unroll
        for (int d = 0; d < TDEPTH; ++d) ld_t(tv[d], d);
#pragma unroll
        for (int j = 0; j < NBUF - 1; ++j) ld_w(wr[j], j);
        st_t(tv[0], 0);
        __syncthreads();
        for (int kb = 0; kb < nfull; kb += U) {
#pragma unroll
          for (int j = 0; j < U; ++j) {
            if (j > 0 && kb + j >= nfull) break;
            ld_t(tv[j % TDEPTH], kb + j + TDEPTH);
            ld_w(wr[(j + NBUF - 1) % NBUF], kb + j + NBUF - 1);
            mm(wr[j % NBUF], (kb + j) & 1, KSTEPS);
            st_t(tv[(j + 1) % TDEPTH], (kb + j + 1) & 1);
            __syncthreads();
          }
        }
      }
      if (tail_steps > 0) {
        const int buf = nfull & 1;
        const int tb = tail_steps * 64;
#pragma unroll
        for (int i = 0; i < NTL; ++i)
          tv[0][i] = ccol < tb ? buffer_load16(tres, toff[i], nfull * KBLK) : u32x4{0u, 0u, 0u, 0u};
        st_t(tv[0], buf);
        const uint32_t o = static_cast<uint32_t>(nfull) * SBLK;
#pragma unroll
        for (int st = 0; st < KSTEPS; ++st)
#pragma unroll
          for (int a = 0; a < NMAT; ++a)
#pragma unroll
            for (int nf = 0; nf < NF; ++nf)
              if (st < tail_steps) wr[0][a][nf][st] = buffer_load16<NTW>(wres[a], woff_v[nf], woff_s[nf] + o + st * SSTEP);
        __syncthreads();
        mm(wr[0], buf, tail_steps);
      }
      epilogue(acc);
    };
    static_assert(MF % kFragGroup == 0, "tile height must be whole fragment groups");
    switch ((mf_active + kFragGroup - 1) / kFragGroup) {
      case 1: run(std::integral_constant<int, kFragGroup>{}); break;
      case 2: run(std::integral_constant<int, 2 * kFragGroup < MF ? 2 * kFragGroup : MF>{}); break;
      case 3: run(std::integral_constant<int, 3 * kFragGroup < MF ? 3 * kFragGroup : MF>{}); break;
      case 4: run(std::integral_constant<int, 4 * kFragGroup < MF ? 4 * kFragGroup : MF>{}); break;
      case 5: run(std::integral_constant<int, 5 * kFragGroup < MF ? 5 * kFragGroup : MF>{}); break;
      case 6: run(std::integral_constant<int, 6 * kFragGroup < MF ? 6 * kFragGroup : MF>{}); break;
      case 7: run(std::integral_constant<int, 7 * kFragGroup < MF ? 7 * kFragGroup : MF>{}); break;
      default: run(std::integral_constant<int, MF>{}); break;
    }
  } else {
    // ---- streaming shapes -----------------------------------------------------
    f32x4 acc[NMAT][NF][MF];
#pragma unroll
    for (int a = 0; a < NMAT; ++a)
#pragma unroll
      for (int nf = 0; nf < NF; ++nf)
#pragma unroll
        for (int mf = 0; mf < MF; ++mf) acc[a][nf][mf] = f32x4{0.f, 0.f, 0.f, 0.f};
    // ---- operand pointers ---------------------------------------------------
    const uint8_t* wrow[NMAT][NF];
#pragma unroll
    for (int nf = 0; nf < NF; ++nf) {
      size_t off;
      if (PACKED) {
        const int frag = min((ncol0 + nf * 16) / 16, N / 16 - 1);
        off = (static_cast<size_t>(frag) * (Kb_row / 64) + kofs / 64) * 1024 + lane * 16;
      } else {
        const int n = min(ncol0 + nf * 16 + lrow, N - 1);
        off = static_cast<size_t>(n) * Kb_row + kofs + lgrp * 16;
      }
      wrow[0][nf] = W0 + off;
      if (SWIGLU) wrow[NMAT - 1][nf] = W1 + off;
    }
    const uint8_t* arow[CPT];
    int acol[CPT], aoff[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = threadIdx.x + i * 256;
      const int r = c / (KBLK / 16);
      acol[i] = (c % (KBLK / 16)) * 16;
      aoff[i] = r * LDS_ROW + acol[i];
      arow[i] = nullptr;
      if (r < nrows) {
        const int grow = row0 + rbeg + r;
        const int src = perm ? perm[grow] : grow;
        arow[i] = A + static_cast<size_t>(src) * lda_b;
      }
    }


    // Loads of K block kb; past the last block (kb >= nfull) every lane reads the same
    // 64 bytes at the start of the first token row instead, which stay in L2, so the
    // ring's tail prefetch costs no memory traffic and the loop needs no branch.
    const uint8_t* dummy = A + (lane & 3) * 16;
    auto load_w = [&](u32x4 (&w)[NMAT][NF][KSTEPS], int kb) {
      const bool real = kb < nfull;
      const size_t off = static_cast<size_t>(real ? kb : 0) * SBLK;
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
        for (int a = 0; a < NMAT; ++a)
#pragma unroll
          for (int nf = 0; nf < NF; ++nf)
            w[a][nf][s] = load_weight<NTW>(real ? wrow[a][nf] + off + s * SSTEP : dummy);
    };
    auto load_a = [&](u32x4 (&av)[CPT], int kb, int bytes) {
      const int off = kb * KBLK;
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        av[i] = u32x4{0u, 0u, 0u, 0u};
        if (arow[i] && acol[i] < bytes) av[i] = *reinterpret_cast<const u32x4*>(arow[i] + off + acol[i]);
      }
    };
    auto store_a = [&](const u32x4 (&av)[CPT], int buf) {
#pragma unroll
      for (int i = 0; i < CPT; ++i) *reinterpret_cast<u32x4*>(&sA[buf][aoff[i]]) = av[i];
    };
    auto step = [&](const u32x4 (&w)[NMAT][NF][KSTEPS], int buf, int s) {
#pragma unroll
      for (int mf = 0; mf < MF; ++mf) {
        if (MF == 1 || mf < mf_active) {
          const u32x4 bfr =
              *reinterpret_cast<const u32x4*>(&sA[buf][(mf * 16 + lrow) * LDS_ROW + s * 64 + lgrp * 16]);
#pragma unroll
          for (int a = 0; a < NMAT; ++a)
#pragma unroll
            for (int nf = 0; nf < NF; ++nf) acc[a][nf][mf] = mfma_chunk<EL>(w[a][nf][s], bfr, acc[a][nf][mf]);
        }
      }
    };
    // E4M3: slices s and s + 1 through one 16x16x128 MFMA (two = false: s is a lone last
    // slice, paired with zeros on both sides)
    auto step2 = [&](const u32x4 (&w)[NMAT][NF][KSTEPS], int buf, int s, bool two) {
      const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int mf = 0; mf < MF; ++mf) {
        if (MF == 1 || mf < mf_active) {
          const uint8_t* bp = &sA[buf][(mf * 16 + lrow) * LDS_ROW + s * 64 + lgrp * 16];
          const u32x4 b0 = *reinterpret_cast<const u32x4*>(bp);
          const u32x4 b1 = two ? *reinterpret_cast<const u32x4*>(bp + 64) : z;
#pragma unroll
          for (int a = 0; a < NMAT; ++a)
#pragma unroll
            for (int nf = 0; nf < NF; ++nf)
              acc[a][nf][mf] = mfma_e4m3_pair(w[a][nf][s], two ? w[a][nf][s + 1] : z, b0, b1, acc[a][nf][mf]);
        }
      }
    };
    constexpr bool kPairs = EL == EL_E4M3 && KSTEPS % 2 == 0;
    auto compute = [&](const u32x4 (&w)[NMAT][NF][KSTEPS], int buf) {
      if constexpr (kPairs) {
#pragma unroll
        for (int s = 0; s < KSTEPS; s += 2) step2(w, buf, s, true);
      } else {
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) step(w, buf, s);
      }
    };

    // Weight ring of NBUF K blocks: block b lives in buffer b % NBUF and is requested
    // NBUF - 1 blocks before it is multiplied.  Prefetches past the last block read the
    // L2-resident dummy instead of being guarded, so the loop body has no data-dependent
    // branches.
    u32x4 wb[NBUF][NMAT][NF][KSTEPS];
    u32x4 av[CPT];
    if (nfull > 0) {
      load_a(av, 0, KBLK);
#pragma unroll
      for (int j = 0; j < NBUF - 1; ++j) load_w(wb[j], j);
      store_a(av, 0);
      __syncthreads();
      for (int kb = 0; kb < nfull; kb += NBUF) {
#pragma unroll
        for (int j = 0; j < NBUF; ++j) {
          if (j > 0 && kb + j >= nfull) break;
          load_a(av, min(kb + j + 1, nfull - 1), KBLK);
          load_w(wb[(j + NBUF - 1) % NBUF], kb + j + NBUF - 1);
          compute(wb[j], (kb + j) & 1);
          store_a(av, (kb + j + 1) & 1);
          __syncthreads();
        }
      }
    }
    if (tail_steps > 0) {
      const int buf = nfull & 1;
      load_a(av, nfull, tail_steps * 64);
      store_a(av, buf);
      const size_t off = static_cast<size_t>(nfull) * SBLK;
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
        for (int a = 0; a < NMAT; ++a)
#pragma unroll
          for (int nf = 0; nf < NF; ++nf)
            if (s < tail_steps) wb[0][a][nf][s] = load_weight<NTW>(wrow[a][nf] + off + s * SSTEP);
      __syncthreads();
      if constexpr (kPairs) {
#pragma unroll
        for (int s = 0; s < KSTEPS; s += 2)
          if (s < tail_steps) step2(wb[0], buf, s, s + 1 < tail_steps);
      } else {
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s)
          if (s < tail_steps) step(wb[0], buf, s);
      }
    }
    epilogue(acc);
  }
#undef SEL
}

// Shape of a launch: tile height, K-block depth, weight ring depth, weight load kind,
// workgroups per CU the register budget is sized for.
// NT: non-temporal weight loads, used where each weight byte is read by one tile and
// the loads cover whole contiguous runs (packed layout); with row-major weights a
// 128-byte line is split over two load instructions, and the hint costs bandwidth.
// stream16 with 16-bit weights: one workgroup per CU and a four-block weight ring
// (three blocks in flight per wave) keeps more bytes in flight than two workgroups with
// a two-block ring; with E4M3 weights two workgroups per CU measured faster.
template <int EL, int SHAPE, bool SWIGLU, bool PACKED> struct Shape;
template <int EL, bool SWIGLU, bool PACKED> struct Shape<EL, kShapeStream16, SWIGLU, PACKED> {
  static constexpr int MF = 1, KSTEPS = SWIGLU ? 8 : 4, TDEPTH = 1;
  static constexpr int NBUF = EL == EL_E4M3 ? 2 : 4, MINB = EL == EL_E4M3 ? 2 : 1;
  static constexpr bool NT = PACKED;
};
template <int EL, bool SWIGLU, bool PACKED> struct Shape<EL, kShapeStream32, SWIGLU, PACKED> {
  static constexpr int MF = 2, KSTEPS = 8, NBUF = 2, MINB = 2, TDEPTH = 1;
  static constexpr bool NT = PACKED;
};
template <int EL, bool SWIGLU, bool PACKED> struct Shape<EL, kShapeTile256, SWIGLU, PACKED> {
  static constexpr int MF = 16, KSTEPS = 2, NBUF = 3, MINB = 1, TDEPTH = 2;
  static constexpr bool NT = PACKED;
};

template <int EL, int OUT, bool SWIGLU, int SHAPE, bool PACKED>
hipError_t launch_one(const GemmProblem& p0, const GemmProblem* p1, int max_tiles0, hipStream_t stream) {
  using S = Shape<EL, SHAPE, SWIGLU, PACKED>;
  constexpr int NF = gemm_nf(SWIGLU, SHAPE);
  constexpr int BM = 16 * S::MF, BN = 4 * NF * 16;
  int tiles1 = 0;
  GemmProblem q1 = p0;
  if (p1) {
    q1 = *p1;
    tiles1 = ((p1->rows + BM - 1) / BM) * p1->k_splits * ((p1->N + BN - 1) / BN);
  }
  const int grid = max_tiles0 + tiles1;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_kernel<EL, OUT, S::MF, NF, SWIGLU, S::KSTEPS, S::NBUF, S::NT, S::MINB, PACKED, S::TDEPTH>),
                     dim3(grid), dim3(256), 0, stream, p0, q1, p1 ? 1 : 0);
  return hipGetLastError();
}

template <int EL, int OUT, bool SWIGLU, bool PACKED>
hipError_t launch_layout(int shape, const GemmProblem& p0, const GemmProblem* p1, int max_tiles0,
                         hipStream_t stream) {
  switch (shape) {
    case kShapeStream16: return launch_one<EL, OUT, SWIGLU, kShapeStream16, PACKED>(p0, p1, max_tiles0, stream);
    case kShapeStream32: return launch_one<EL, OUT, SWIGLU, kShapeStream32, PACKED>(p0, p1, max_tiles0, stream);
    default: return launch_one<EL, OUT, SWIGLU, kShapeTile256, PACKED>(p0, p1, max_tiles0, stream);
  }
}

template <int EL, int OUT, bool SWIGLU>
hipError_t launch_shape(int shape, bool packed, const GemmProblem& p0, const GemmProblem* p1, int max_tiles0,
                        hipStream_t stream) {
  return packed ? launch_layout<EL, OUT, SWIGLU, true>(shape, p0, p1, max_tiles0, stream)
                : launch_layout<EL, OUT, SWIGLU, false>(shape, p0, p1, max_tiles0, stream);
}

}  // namespace

hipError_t launch_gemm(int el, int out_el, bool swiglu, int shape, bool packed, const GemmProblem& p0,
                       const GemmProblem* p1, int max_tiles0, hipStream_t stream) {
#define MOE_GEMM(E_, O_, S_) \
  return launch_shape<E_, O_, S_>(shape, packed, p0, p1, max_tiles0, stream)
  if (swiglu) {
    if (el == EL_F32 && out_el == EL_F32) MOE_GEMM(EL_F32, EL_F32, true);
    if (el == EL_BF16 && out_el == EL_BF16) MOE_GEMM(EL_BF16, EL_BF16, true);
    if (el == EL_E4M3 && out_el == EL_BF16) MOE_GEMM(EL_E4M3, EL_BF16, true);
  } else {
    if (el == EL_F32 && out_el == EL_F32) MOE_GEMM(EL_F32, EL_F32, false);
    if (el == EL_BF16 && out_el == EL_BF16) MOE_GEMM(EL_BF16, EL_BF16, false);
    if (el == EL_BF16 && out_el == EL_F32) MOE_GEMM(EL_BF16, EL_F32, false);
    if (el == EL_E4M3 && out_el == EL_BF16) MOE_GEMM(EL_E4M3, EL_BF16, false);
    if (el == EL_E4M3 && out_el == EL_F32) MOE_GEMM(EL_E4M3, EL_F32, false);
  }
#undef MOE_GEMM
  return hipErrorInvalidValue;
}

}  // namespace moe
