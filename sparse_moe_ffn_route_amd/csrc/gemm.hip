// Ragged grouped GEMM of the expert FFNs (and the router projection), gfx950 MFMA.
//
// Source: the "Grouped GEMMs" block of "Systems Engineering Playbook: Qwen 3.5 MoE on
// Ironwood TPU" (introduction and table "Three High-Leverage Optimizations"); the
// SwiGLU form of the experts is this library's reading of "3. Sparse
// Mixture-of-Experts (MoE)" in "Tối ưu hóa mô hình Qwen 3.5-397B MoE trên hạ tầng TPU
// Ironwood", whose formula is missing.
//
// Work unit (one workgroup of NW waves: 4, or 8 for the router projection's tiles): one
// (group, N-tile, M-tile).  The M-tile is up to 16 * MF token rows of the group (gathered
// through perm); the N-tile is NW waves x NF x 16 output channels (for SwiGLU the same
// channels of W_gate and W_up, so silu(gate) * up is formed in registers).
//
// Data path:
//   * weights go straight from HBM into VGPRs as the MFMA "A" operand; each wave owns
//     its own output channels, so weights are never shared between waves and need no
//     LDS.  Lane l of a wave reads 16 bytes of channel (l % 16) at K-byte offset
//     (l / 16) * 16, so one wave step covers 16 rows x 64 contiguous bytes; K blocks
//     of KSTEPS steps rotate through a ring of NBUF register buffers, so the loads of
//     the next NBUF - 1 blocks are in flight while one block is multiplied.  They are
//     buffer loads (a wave-uniform resource and offset plus one fixed offset per lane),
//     so the loop computes no per-lane addresses and no load waits on a register that
//     the compiler took from a pending load;
//   * token rows are the MFMA "B" operand, shared by the workgroup's waves: staged per K block in
//     LDS, one barrier per block.  The streaming shapes load them into registers and
//     store them to two LDS buffers; the tile shape loads them straight into TDEPTH + 1
//     LDS buffers, TDEPTH blocks ahead (no registers, no LDS store instructions).  Token
//     loads go out before the weights of the same block, so waiting for them never waits
//     for the weight stream;
//   * 16-row token fragments past the tile's last row are skipped (uniform branch), so
//     a ragged group costs MFMA time in 16-row steps only.
// Two shapes are instantiated: a streaming shape (MF = 1 or 2, a ring of two to four K
// blocks; the down projection takes 4 fragments per wave to double the channels each
// workgroup streams) for the few-rows-per-expert decode regime, where
// each weight byte feeds one tile and the kernel is an HBM stream; and a tile shape
// (MF = 16, 2-step blocks, a four-block weight ring and four LDS token buffers, 2
// fragments per matrix per wave, one workgroup per CU so a wave may hold 512 registers;
// the expert down projections take two workgroups per CU with two-block rings) for the
// prefill regime: a 256-row
// M-tile covers every row of a typical expert (~160 at 8K tokens), so each weight byte
// is streamed from HBM once and feeds all of the expert's rows, and 32 channels per
// matrix per wave halve the token bytes staged per MFMA; only experts with more rows
// (skewed routing) take several M-tiles, adjacent in the launch order.
// Tiles are ordered (group, N-tile, M-tile) and dealt to XCDs in contiguous ranges.
#include <type_traits>

#include "common.hpp"
#include "gemm.hpp"

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

// One tile's coordinates and operand bases (wave-uniform).
struct TileInfo {
  int g, row0;               // group, and its first row in the grouped order
  int n_tile, ks;            // N-tile, K split
  int rbeg, nrows;           // first row of the M-tile within the group, rows in use
  int N, Kb_row, Kb, kofs;   // output width; bytes per weight row, per K range; K range offset
  int nfull, tail_steps;     // full K blocks; 64-byte steps of a last partial block
  const uint8_t* A;          // token rows (K range offset applied)
  const int32_t* perm;
  size_t lda_b;
  const uint8_t* W0;
  const uint8_t* W1;
};

// COMB: the epilogue is the fused unpermute-combine of a single-group problem (see
// GemmProblem::comb_rows), instantiated for the shared expert's down projection only.
template <int EL, int OUT, int MF, int NF, bool SWIGLU, int KSTEPS, int NBUF, bool NTW, int MINB, bool PACKED,
          int TDEPTH, bool COMB, int NW>
__global__ __launch_bounds__(NW * 64, MINB) void gemm_kernel(GemmProblem p) {
  constexpr int ES = ElSize<EL>::v;
  constexpr int BM = 16 * MF;
  constexpr int NMAT = SWIGLU ? 2 : 1;
  constexpr int NTHR = NW * kWave;    // threads per workgroup
  constexpr int BN = NW * NF * 16;
  constexpr int KBLK = KSTEPS * 64;   // bytes of each row per K block
  constexpr int LDS_ROW = KBLK + 16;  // padded LDS row (bytes)
  constexpr int CHUNKS = BM * (KBLK / 16);
  static_assert(CHUNKS % NTHR == 0, "token tile must split evenly over the threads");
  constexpr int CPT = CHUNKS / NTHR;  // 16-byte token chunks per thread per K block
  // LDS token staging.  Streaming shapes: two buffers of padded rows (LDS_ROW bytes)
  // written from registers.  Tile shape: TDEPTH + 1 buffers of unpadded KBLK-byte rows in
  // a swizzled chunk order, filled by direct buffer-to-LDS loads.
  constexpr int NLB = MF >= 8 ? TDEPTH + 1 : 2;
  constexpr int SA_BUF = MF >= 8 ? BM * KBLK : BM * LDS_ROW;  // bytes per buffer
  __shared__ __attribute__((aligned(16))) uint8_t sA_lds[NLB * SA_BUF];
  auto sA = [&](int buf) -> uint8_t* { return sA_lds + buf * SA_BUF; };

  // ---- tiles ----------------------------------------------------------------
  const int n_tiles = (p.N + BN - 1) / BN;
  const int total = (p.offsets ? ld_scalar(p.tile_prefix + p.n_groups) : (p.rows + BM - 1) / BM * p.k_splits) * n_tiles;
  // Tile L of the launch order (ordered (group, N-tile, M-tile) within each problem).
  auto locate = [&](int L) {
    TileInfo t;
    const int32_t* offsets = p.offsets;
    int g = 0, row0 = 0, count = p.rows, n_tile, m, ks = 0;
    const int ksp = p.k_splits;
    if (offsets) {
      // group g owns tiles [pre[g] * n_tiles, pre[g + 1] * n_tiles), ordered (N-tile, M-tile)
      const int32_t* pre = p.tile_prefix;
      const int q = L / n_tiles;
      int lo = 0, hi = p.n_groups - 1;
      while (lo < hi) {  // largest g with pre[g] <= q
        const int mid = (lo + hi + 1) >> 1;
        if (ld_scalar(pre + mid) <= q) lo = mid; else hi = mid - 1;
      }
      g = lo;
      const int pg = ld_scalar(pre + g);
      const int mt = ld_scalar(pre + g + 1) - pg;
      const int local = L - pg * n_tiles;
      n_tile = local / mt;
      m = local % mt;
      row0 = ld_scalar(offsets + g);
      count = ld_scalar(offsets + g + 1) - row0;
    } else {
      const int mt = (count + BM - 1) / BM;
      m = L % mt;
      ks = (L / mt) % ksp;
      n_tile = L / mt / ksp;
    }
    // the tile coordinates are wave-uniform; say so, so that addresses built from them
    // stay in scalar registers
    t.g = __builtin_amdgcn_readfirstlane(g);
    t.row0 = __builtin_amdgcn_readfirstlane(row0);
    count = __builtin_amdgcn_readfirstlane(count);
    t.n_tile = __builtin_amdgcn_readfirstlane(n_tile);
    m = __builtin_amdgcn_readfirstlane(m);
    t.ks = __builtin_amdgcn_readfirstlane(ks);
    t.rbeg = m * BM;
    t.nrows = min(BM, count - t.rbeg);
    t.N = p.N;
    t.Kb_row = p.K * ES;               // bytes per row
    t.Kb = t.Kb_row / ksp;             // bytes of this K range
    t.kofs = t.ks * t.Kb;
    t.A = static_cast<const uint8_t*>(p.a) + t.kofs;
    t.perm = p.perm;
    t.lda_b = static_cast<size_t>(p.lda) * ES;
    const size_t wgrp = static_cast<size_t>(t.g) * p.w_stride * ES;
    t.W0 = static_cast<const uint8_t*>(p.w0) + wgrp;
    t.W1 = SWIGLU ? static_cast<const uint8_t*>(p.w1) + wgrp : nullptr;
    // Full K blocks run a branch-free pipeline; a last partial block (K*ES not a
    // multiple of KBLK) is handled after it with per-step guards.
    t.nfull = t.Kb / KBLK;
    t.tail_steps = (t.Kb - t.nfull * KBLK) / 64;
    return t;
  };
  // Weight addressing: row-major rows are Kb_row apart and a 64-byte step is 64 bytes on;
  // in the packed layout a 16-row fragment is one run of 1 KB per step.
  constexpr int SSTEP = PACKED ? 1024 : 64;     // bytes between consecutive 64-byte K steps
  constexpr int SBLK = KSTEPS * SSTEP;          // bytes between consecutive K blocks

  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int lrow = lane & 15, lgrp = lane >> 4;

  // ---- epilogue: scales, SwiGLU, store --------------------------------------
  auto epilogue = [&](const TileInfo& t, const f32x4 (&acc)[NMAT][NF][MF]) {
    void* out = static_cast<uint8_t*>(p.out) + static_cast<size_t>(t.ks) * p.out_split_stride * (OUT == EL_F32 ? 4 : 2);
    const size_t ldo = p.ldo;
    const float* a_scale = p.a_scale;
    const float* s0 = p.s0;
    const float* s1 = p.s1;
    const int N = t.N;
    const int ncol0 = t.n_tile * BN + wave * NF * 16;
#pragma unroll
    for (int mf = 0; mf < MF; ++mf) {
      const int r = mf * 16 + lrow;
      if (r >= t.nrows) continue;
      const int grow = t.row0 + t.rbeg + r;
      float as = 1.0f;
      if (EL == EL_E4M3) as = a_scale[t.perm ? t.perm[grow] : grow];
#pragma unroll
      for (int nf = 0; nf < NF; ++nf) {
        const int n = ncol0 + nf * 16 + lgrp * 4;
        if (n >= N) continue;
        const int valid = min(4, N - n);
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float x0 = acc[0][nf][mf][i];
          if (EL == EL_E4M3) x0 *= as * s0[static_cast<size_t>(t.g) * N + min(n + i, N - 1)];
          if (SWIGLU) {
            float x1 = acc[NMAT - 1][nf][mf][i];
            if (EL == EL_E4M3) x1 *= as * s1[static_cast<size_t>(t.g) * N + min(n + i, N - 1)];
            v[i] = silu(x0) * x1;
          } else {
            v[i] = x0;
          }
        }
        OutStore<OUT>::store4(out, static_cast<size_t>(grow) * ldo + n, v, valid);
      }
    }
  };

  // ---- fused combine epilogue ---------------------------------------------------
  // In passes of PR rows: the tile's fp32 results are staged in LDS (reusing the token
  // buffers), and the pass's slot indices and routing weights are loaded into LDS by the
  // whole workgroup in one coalesced sweep.  Each thread then owns 8 columns of R rows and
  // issues the loads of all R rows' slots in batches (LOADS 16-byte loads in flight), so a
  // pass costs a few memory round trips rather than a few per row; every row's sum still
  // runs over its slots in order: y = sum_j w[t][j] * comb_rows[inv[t][j]] + staged value,
  // rounded once.
  auto epilogue_combine = [&](const TileInfo& t, const f32x4 (&acc)[NMAT][NF][MF]) {
    if constexpr (COMB) {
      constexpr int SROW = BN + 4;                          // floats per staged row (16-byte pad)
      constexpr int KMAX = 32;                              // largest top_k the library accepts
      constexpr int LDS_BYTES = NLB * SA_BUF;
      constexpr int ROW_BYTES = SROW * 4 + KMAX * 8;        // staged row + its slot indices and weights
      constexpr int PR1 = (LDS_BYTES / ROW_BYTES) / 16 * 16;
      constexpr int PR2 = PR1 < BM ? PR1 : BM;
      constexpr int PR = PR2 >= 64 && BM % 64 == 0 ? 64 : PR2 >= 32 && BM % 32 == 0 ? 32 : 16;  // rows per pass
      static_assert(PR * ROW_BYTES <= LDS_BYTES && BM % PR == 0, "combine staging pass must fit the LDS");
      constexpr int TPR = BN / 8;                           // threads per row (8 columns each)
      constexpr int RPI = NTHR / TPR;                       // rows per workgroup sweep
      constexpr int R = PR / RPI;                           // rows per thread per pass
      static_assert(R >= 1 && PR % RPI == 0, "rows per pass must split evenly over the threads");
      constexpr int PIECES = OUT == EL_F32 ? 2 : 1;         // 16-byte loads per 8-column piece
      constexpr int LOADS = 20 / PIECES;                    // pieces in flight per thread
      constexpr int KB = LOADS / R > 0 ? LOADS / R : 1;     // slots per batch
      float* st = reinterpret_cast<float*>(sA(0));
      int32_t* s_inv = reinterpret_cast<int32_t*>(st + PR * SROW);
      float* s_w = reinterpret_cast<float*>(s_inv + PR * KMAX);
      const int N = t.N, k = p.comb_k;
      const int cw = wave * NF * 16;
      const int cc = (threadIdx.x % TPR) * 8;
      const int n = t.n_tile * BN + cc;
      const int r0 = threadIdx.x / TPR;
      const size_t ldo = p.ldo;
      typedef typename std::conditional<OUT == EL_F32, float, uint16_t>::type OutT;
      const OutT* rows_src = static_cast<const OutT*>(p.comb_rows);
      OutT* out = static_cast<OutT*>(p.out);
#pragma unroll
      for (int pass = 0; pass < BM / PR; ++pass) {
        __syncthreads();  // the K loop's last LDS reads (or the previous pass) are done
#pragma unroll
        for (int m = 0; m < PR / 16; ++m) {
          const int mf = pass * (PR / 16) + m;
#pragma unroll
          for (int nf = 0; nf < NF; ++nf)
            *reinterpret_cast<f32x4*>(&st[(m * 16 + lrow) * SROW + cw + nf * 16 + lgrp * 4]) = acc[0][nf][mf];
        }
        // the pass's rows are tokens tok0 .. tok0 + rows - 1: their k slot indices are one
        // contiguous run of inv, their weights plane 1 of each token's blob
        const int rows = min(PR, t.nrows - pass * PR);
        const int tok0 = t.row0 + t.rbeg + pass * PR;
        for (int q = threadIdx.x; q < rows * k; q += NTHR) {
          const int r = q / k, j = q - r * k;
          s_inv[r * KMAX + j] = p.comb_inv[static_cast<size_t>(tok0) * k + q];
          s_w[r * KMAX + j] = __int_as_float(p.comb_packed[(static_cast<size_t>(tok0) + r) * 2 * k + k + j]);
        }
        __syncthreads();
        if (n < N && r0 < rows) {
          float a[R][8];
#pragma unroll
          for (int i = 0; i < R; ++i)
#pragma unroll
            for (int q = 0; q < 8; ++q) a[i][q] = 0.f;
          for (int j0 = 0; j0 < k; j0 += KB) {
            int ri[R][KB];
            u32x4 v[R][KB][PIECES];
#pragma unroll
            for (int i = 0; i < R; ++i)
#pragma unroll
              for (int u = 0; u < KB; ++u) {
                const int rr = r0 + i * RPI;
                ri[i][u] = (rr < rows && j0 + u < k) ? s_inv[rr * KMAX + j0 + u] : -1;
              }
            // Unconditional loads: a missing slot (not local, or past k) reads row 0, which is
            // never summed.  With the loads under per-slot branches the compiler waited for each
            // load before issuing the next.
#pragma unroll
            for (int i = 0; i < R; ++i)
#pragma unroll
              for (int u = 0; u < KB; ++u) {
                const OutT* src = rows_src + static_cast<size_t>(ri[i][u] < 0 ? 0 : ri[i][u]) * ldo + n;
#pragma unroll
                for (int c = 0; c < PIECES; ++c) v[i][u][c] = reinterpret_cast<const u32x4*>(src)[c];
              }
#pragma unroll
            for (int i = 0; i < R; ++i)
#pragma unroll
              for (int u = 0; u < KB; ++u) {
                if (ri[i][u] < 0) continue;
                const float w = s_w[(r0 + i * RPI) * KMAX + j0 + u];
                float x[8];
                if constexpr (OUT == EL_F32) {
#pragma unroll
                  for (int q = 0; q < 4; ++q) {
                    x[q] = __uint_as_float(v[i][u][0][q]);
                    x[4 + q] = __uint_as_float(v[i][u][PIECES - 1][q]);
                  }
                } else {
#pragma unroll
                  for (int q = 0; q < 4; ++q) {
                    x[2 * q] = bf16_bits_to_f32(v[i][u][0][q] & 0xFFFFu);
                    x[2 * q + 1] = bf16_bits_to_f32(v[i][u][0][q] >> 16);
                  }
                }
#pragma unroll
                for (int q = 0; q < 8; ++q) a[i][q] = fmaf(w, x[q], a[i][q]);
              }
          }
#pragma unroll
          for (int i = 0; i < R; ++i) {
            const int rr = r0 + i * RPI;
            if (rr >= rows) break;
            const float* sv = &st[rr * SROW + cc];
            float o[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) o[q] = a[i][q] + sv[q];
            OutT* dst = out + static_cast<size_t>(tok0 + rr) * ldo + n;
            if constexpr (OUT == EL_F32) {
              reinterpret_cast<float4*>(dst)[0] = make_float4(o[0], o[1], o[2], o[3]);
              reinterpret_cast<float4*>(dst)[1] = make_float4(o[4], o[5], o[6], o[7]);
            } else {
              *reinterpret_cast<uint4*>(dst) = make_uint4(bf16x2_bits(o[0], o[1]), bf16x2_bits(o[2], o[3]),
                                                          bf16x2_bits(o[4], o[5]), bf16x2_bits(o[6], o[7]));
            }
          }
        }
      }
    }
  };
  auto finish = [&](const TileInfo& t, const f32x4 (&acc)[NMAT][NF][MF]) {
    if constexpr (COMB) epilogue_combine(t, acc);
    else epilogue(t, acc);
  };

  if constexpr (MF >= 8) {
    // ---- tile shape ---------------------------------------------------------
    if (static_cast<int>(blockIdx.x) >= total) return;
    const TileInfo ti = locate(xcd_remap(blockIdx.x, total));
    const int N = ti.N, Kb_row = ti.Kb_row, kofs = ti.kofs;
    const int row0 = ti.row0, rbeg = ti.rbeg, nrows = ti.nrows, n_tile = ti.n_tile;
    const int nfull = ti.nfull, tail_steps = ti.tail_steps;
    const int32_t* perm = ti.perm;
    const size_t lda_b = ti.lda_b;
    const uint8_t* A = ti.A;
    const uint8_t* W0 = ti.W0;
    const uint8_t* W1 = ti.W1;
    const int mf_active = (nrows + 15) / 16;
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
    static_assert(CPR == 8, "tile shape: 128-byte K blocks");
    constexpr int RPP = NTHR / CPR;       // token rows per pass of the workgroup (NW KB)
    constexpr int NTP = BM / RPP;         // passes for a full tile
    // Token rows go from memory straight into LDS (buffer loads with the LDS as
    // destination: no registers, no LDS store instructions).  An LDS row is the K block's
    // KBLK bytes, unpadded, with the row's 16-byte chunk c at chunk slot c ^ ((r >> 1) & 7):
    // the 16 rows of a fragment read at one column then fall into 16 different bank
    // groups.  A direct load writes 16 bytes per lane at the wave's LDS base plus 16 * lane,
    // so lane l of wave w fills slot (32 i + 8 w + l / 8, l % 8) in pass i and loads the
    // chunk of that row that belongs there.
    const int crow = threadIdx.x / CPR;
    const int ccol = ((threadIdx.x % CPR) ^ ((crow >> 1) & 7)) * 16;
    const __amdgpu_buffer_rsrc_t tres = buffer_rsrc(A);
    const __amdgpu_buffer_rsrc_t none = buffer_rsrc_empty();
    uint32_t toff[NTP];
#pragma unroll
    for (int i = 0; i < NTP; ++i) {
      const int grow = row0 + rbeg + min(crow + i * RPP, nrows - 1);
      toff[i] = static_cast<uint32_t>(perm ? perm[grow] : grow) * static_cast<uint32_t>(lda_b) + ccol;
    }
    // a lane's fragment reads: row lrow of each 16-row fragment, chunk 4 * step + lgrp
    uint32_t rd_off[KSTEPS];
#pragma unroll
    for (int st = 0; st < KSTEPS; ++st) rd_off[st] = lrow * KBLK + (((st * 4 + lgrp) ^ ((lrow >> 1) & 7)) * 16);

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
      // weights of block kb (past the last block: the empty resource, no memory touched)
      auto ld_w = [&](u32x4 (&w)[NMAT][NF][KSTEPS], int kb) {
        const bool real = kb < nfull;
        const uint32_t o = static_cast<uint32_t>(real ? kb : 0) * SBLK;
#pragma unroll
        for (int st = 0; st < KSTEPS; ++st)
#pragma unroll
          for (int a = 0; a < NMAT; ++a)
#pragma unroll
            for (int nf = 0; nf < NF; ++nf)
              w[a][nf][st] = buffer_load16<NTW>(real ? wres[a] : none, woff_v[nf], woff_s[nf] + o + st * SSTEP);
      };
      // token rows of block kb into LDS buffer buf (past the last block: empty resource)
      auto ld_t = [&](int buf, int kb) {
        const bool real = kb < nfull;
        const uint32_t o = static_cast<uint32_t>(real ? kb : 0) * KBLK;
        uint8_t* dst = sA(buf) + wv * 1024;
#pragma unroll
        for (int i = 0; i < NTL; ++i)
          buffer_load16_to_lds(real ? tres : none, dst + i * RPP * KBLK, toff[i], o);
      };
      // Token fragments are read kLdsAhead fragments ahead of the MFMAs that use them
      // (a ring of kLdsAhead + 1 registers); the scheduling barriers keep that order
      // (the scheduler would otherwise hoist every read of the block and run out of
      // registers).
      constexpr int kLdsAhead = 1;
      constexpr int NQ = kLdsAhead + 1;
      auto mm = [&](const u32x4 (&w)[NMAT][NF][KSTEPS], int buf, int nst) {
        const uint8_t* sb = sA(buf);
        const int total = nst * MFR;  // (step, fragment) pairs of this block, in issue order
        auto frag_at = [&](int q) {
          return *reinterpret_cast<const u32x4*>(sb + (q % MFR) * 16 * KBLK + rd_off[q / MFR]);
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
      // Block b's token rows are requested TD = TDEPTH blocks ahead into LDS buffer
      // b % NLB, just before block b + NBUF - 1's weights; at the end of block b each wave
      // waits for its own part of block b + 1's rows and the workgroup meets at a barrier,
      // after which every wave may read them.  Vector loads complete in issue order, so
      // that wait allows exactly the loads issued after those rows to stay in flight (the
      // weights issued with them and the TD - 1 blocks after); it never waits for weights
      // still to be used.  The barrier is the bare instruction: a workgroup fence here would
      // wait for every load in flight, since LDS-bound loads are outstanding.  Buffer
      // b % NLB is refilled at block b + NLB - TD = b + 1, after the barrier that ends
      // block b.  The loop is unrolled over lcm(NBUF, NLB) blocks so that the ring indices
      // are compile-time constants.
      constexpr int TD = TDEPTH;
      static_assert(NLB == TD + 1 && NBUF - 1 >= TD, "token lead within the LDS and weight rings");
      constexpr int WL = NMAT * NF * KSTEPS;              // weight loads per block per lane
      constexpr int kAfter = WL + (TD - 1) * (NTL + WL);  // loads issued after block b + 1's rows
      constexpr int kWait = kAfter < 63 ? kAfter : 63;
      auto wait_rows = [&]() { wait_vmcnt<kWait>(); };
      auto barrier = [&]() { bare_barrier(); };
      constexpr int U = NBUF * NLB / gcd_c(NBUF, NLB);
      if (nfull > 0) {
        // the prologue issues TD blocks of rows, then NBUF - 1 >= TD blocks of weights, so
        // at least kAfter loads follow block 0's rows
#pragma unroll
        for (int d = 0; d < TD; ++d) ld_t(d, d);
        // the wait counts rely on this issue order: keep the scheduler from mixing them
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < NBUF - 1; ++j) ld_w(wr[j], j);
        __builtin_amdgcn_sched_barrier(0);
        wait_rows();
        barrier();
        for (int kb = 0; kb < nfull; kb += U) {
#pragma unroll
          for (int j = 0; j < U; ++j) {
            if (j > 0 && kb + j >= nfull) break;
            ld_t((j + TD) % NLB, kb + j + TD);
            __builtin_amdgcn_sched_barrier(0);
            ld_w(wr[(j + NBUF - 1) % NBUF], kb + j + NBUF - 1);
            __builtin_amdgcn_sched_barrier(0);
            mm(wr[j % NBUF], j % NLB, KSTEPS);
            __builtin_amdgcn_sched_barrier(0);
            wait_rows();
            barrier();
          }
        }
      }
      // Loads still in flight (past the last block) read through the empty resource; the
      // LDS-bound ones must land before the LDS is used again or the workgroup ends.
      wait_vmcnt<0>();
      if (tail_steps > 0) {
        // a last partial K block: token rows through registers with a guard per chunk,
        // stored to the same swizzled slots
        const int buf = nfull % NLB;
        const int tb = tail_steps * 64;
#pragma unroll
        for (int i = 0; i < NTL; ++i) {
          const u32x4 v = ccol < tb ? buffer_load16(tres, toff[i], nfull * KBLK) : u32x4{0u, 0u, 0u, 0u};
          *reinterpret_cast<u32x4*>(sA(buf) + i * RPP * KBLK + threadIdx.x * 16) = v;
        }
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
      finish(ti, acc);
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
    if (static_cast<int>(blockIdx.x) >= total) return;
    const TileInfo ti = locate(xcd_remap(blockIdx.x, total));
    const int nfull = ti.nfull, tail_steps = ti.tail_steps;
    const int mf_active = (ti.nrows + 15) / 16;
    static_assert(NBUF >= 2 && NBUF <= 4, "streaming ring of 2 to 4 blocks");
    static_assert(NW == 4, "streaming shapes: 4 waves");

    // Weights as buffer loads: a resource per matrix at the group's weights, a fixed
    // 32-bit offset per lane and fragment, and a wave-uniform offset per fragment to which
    // the K-block offset is added.  The ring's loads then need no per-lane address
    // arithmetic and no registers beyond their destinations, so the compiler never takes
    // a pending load's registers for an address (which would wait for that load).
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    __amdgpu_buffer_rsrc_t wres[NMAT];
    wres[0] = buffer_rsrc(ti.W0);
    if (SWIGLU) wres[NMAT - 1] = buffer_rsrc(ti.W1);
    uint32_t wvo[NF], wso[NF];
    {
      const int ncol0 = ti.n_tile * BN + wv * NF * 16;
#pragma unroll
      for (int nf = 0; nf < NF; ++nf) {
        if (PACKED) {
          const int frag = min((ncol0 + nf * 16) / 16, ti.N / 16 - 1);
          wso[nf] = (static_cast<uint32_t>(frag) * (ti.Kb_row / 64) + ti.kofs / 64) * 1024;
          wvo[nf] = lane * 16;
        } else {
          const int n = min(ncol0 + nf * 16 + lrow, ti.N - 1);
          wso[nf] = ti.kofs;
          wvo[nf] = static_cast<uint32_t>(n) * ti.Kb_row + lgrp * 16;
        }
      }
    }
    // Token chunks: thread -> (row in the tile, byte column); rows past the tile's last
    // row re-read that row (their output rows are never stored), so every token load is
    // unconditional.  Token rows stay 64-bit addressed: this shape also serves inputs
    // past 2 GiB.
    const uint8_t* arow[CPT];
    int acol[CPT], aoff[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = threadIdx.x + i * NTHR;
      const int r = c / (KBLK / 16);
      acol[i] = (c % (KBLK / 16)) * 16;
      aoff[i] = r * LDS_ROW + acol[i];
      const int grow = ti.row0 + ti.rbeg + min(r, ti.nrows - 1);
      const int src = ti.perm ? ti.perm[grow] : grow;
      arow[i] = ti.A + static_cast<size_t>(src) * ti.lda_b;
    }
    // Prefetches past the last block go through an empty resource: they return zeros
    // without touching memory, so the ring's tail needs no branch.
    const __amdgpu_buffer_rsrc_t none = buffer_rsrc_empty();

    auto load_w = [&](u32x4 (&w)[NMAT][NF][KSTEPS], int kb) {
      const bool real = kb < nfull;
      const uint32_t off = static_cast<uint32_t>(real ? kb : 0) * SBLK;
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
        for (int a = 0; a < NMAT; ++a)
#pragma unroll
          for (int nf = 0; nf < NF; ++nf)
            w[a][nf][s] = buffer_load16<NTW>(real ? wres[a] : none, wvo[nf], wso[nf] + off + s * SSTEP);
    };
    auto load_a = [&](u32x4 (&av)[CPT], int kb) {
      const int off = kb * KBLK;
#pragma unroll
      for (int i = 0; i < CPT; ++i) av[i] = *reinterpret_cast<const u32x4*>(arow[i] + off + acol[i]);
    };
    auto store_a = [&](const u32x4 (&av)[CPT], int buf) {
#pragma unroll
      for (int i = 0; i < CPT; ++i) *reinterpret_cast<u32x4*>(sA(buf) + aoff[i]) = av[i];
    };
    f32x4 acc[NMAT][NF][MF];
#pragma unroll
    for (int a = 0; a < NMAT; ++a)
#pragma unroll
      for (int nf = 0; nf < NF; ++nf)
#pragma unroll
        for (int mf = 0; mf < MF; ++mf) acc[a][nf][mf] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto step = [&](const u32x4 (&w)[NMAT][NF][KSTEPS], int buf, int s) {
#pragma unroll
      for (int mf = 0; mf < MF; ++mf) {
        if (MF == 1 || mf < mf_active) {
          const u32x4 bfr =
              *reinterpret_cast<const u32x4*>(sA(buf) + (mf * 16 + lrow) * LDS_ROW + s * 64 + lgrp * 16);
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
          const uint8_t* bp = sA(buf) + (mf * 16 + lrow) * LDS_ROW + s * 64 + lgrp * 16;
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
    // NBUF - 1 blocks before it is multiplied; token rows of block b + 1 are staged in LDS
    // buffer (b + 1) & 1 while block b is multiplied.
    u32x4 wb[NBUF][NMAT][NF][KSTEPS];
    u32x4 av[CPT];
    if (nfull > 0) {
      load_a(av, 0);
#pragma unroll
      for (int j = 0; j < NBUF - 1; ++j) load_w(wb[j], j);
      store_a(av, 0);
      __syncthreads();
      // Whole ring turns, then a part turn of the blocks left over.  A whole turn has no
      // exit inside, so at the top of the loop every load of the previous turn is known to
      // have been consumed and nothing there waits for the loads still in flight.  The
      // token loads of a block go out before its weight loads: the wait for them at the
      // end of the block then leaves the block's weight loads in flight.
      auto block = [&](auto jc, int kb) {
        constexpr int j = decltype(jc)::value;
        load_a(av, min(kb + j + 1, nfull - 1));
        __builtin_amdgcn_sched_barrier(0);
        load_w(wb[(j + NBUF - 1) % NBUF], kb + j + NBUF - 1);
        compute(wb[j], (kb + j) & 1);
        store_a(av, (kb + j + 1) & 1);
        __syncthreads();
      };
      const int kb_full = nfull - nfull % NBUF;
      int kb = 0;
      for (; kb < kb_full; kb += NBUF) {
        block(std::integral_constant<int, 0>{}, kb);
        block(std::integral_constant<int, 1>{}, kb);
        if constexpr (NBUF > 2) block(std::integral_constant<int, 2>{}, kb);
        if constexpr (NBUF > 3) block(std::integral_constant<int, 3>{}, kb);
      }
      if (kb < nfull) {
        block(std::integral_constant<int, 0>{}, kb);
        if (kb + 1 < nfull) block(std::integral_constant<int, 1>{}, kb);
        if constexpr (NBUF > 2) if (kb + 2 < nfull) block(std::integral_constant<int, 2>{}, kb);
        if constexpr (NBUF > 3) if (kb + 3 < nfull) block(std::integral_constant<int, 3>{}, kb);
      }
    }
    if (tail_steps > 0) {
      // a last partial K block: per-step guards
      const int buf = nfull & 1;
      const int tb = tail_steps * 64;
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        av[i] = u32x4{0u, 0u, 0u, 0u};
        if (acol[i] < tb) av[i] = *reinterpret_cast<const u32x4*>(arow[i] + nfull * KBLK + acol[i]);
      }
      store_a(av, buf);
      const uint32_t off = static_cast<uint32_t>(nfull) * SBLK;
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
        for (int a = 0; a < NMAT; ++a)
#pragma unroll
          for (int nf = 0; nf < NF; ++nf)
            if (s < tail_steps) wb[0][a][nf][s] = buffer_load16<NTW>(wres[a], wvo[nf], wso[nf] + off + s * SSTEP);
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
    finish(ti, acc);
  }
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
// tile256 down projections of the experts (E4M3, or packed 16-bit weights; the router
// projection keeps its row-major shape): K is short (I = 1024), so a tile runs few K
// blocks and its prologue and epilogue weigh; 2 fragments per wave, a two-block ring
// and one block of token lookahead fit two workgroups per CU, which overlap one
// another's ends (for e4m3 the compiler keeps four 64-bit values in scratch outside the
// K loop; one workgroup per CU with 4 fragments per wave measured slower for both).
template <int EL, bool SWIGLU, bool PACKED> struct Shape<EL, kShapeTile256, SWIGLU, PACKED> {
  static constexpr bool kTwoPerCu = !SWIGLU && (EL == EL_E4M3 || PACKED);
  static constexpr int MF = 16, KSTEPS = 2, NBUF = kTwoPerCu ? 2 : 4, MINB = kTwoPerCu ? 2 : 1;
  static constexpr int TDEPTH = kTwoPerCu ? 1 : 3;  // token rows' lead; TDEPTH + 1 LDS buffers
  static constexpr bool NT = PACKED;
};

template <int EL, int OUT, bool SWIGLU, int SHAPE, bool PACKED, bool COMB = false>
hipError_t launch_one(const GemmProblem& p, int max_tiles, hipStream_t stream) {
  using S = Shape<EL, SHAPE, SWIGLU, PACKED>;
  constexpr int NF = gemm_nf(SWIGLU, SHAPE, EL, PACKED);
  constexpr int NW = gemm_nw(SWIGLU, SHAPE, EL, PACKED);
  if (max_tiles == 0) return hipSuccess;
  hipLaunchKernelGGL(
      (gemm_kernel<EL, OUT, S::MF, NF, SWIGLU, S::KSTEPS, S::NBUF, S::NT, S::MINB, PACKED, S::TDEPTH, COMB, NW>),
      dim3(max_tiles), dim3(NW * 64), 0, stream, p);
  return hipGetLastError();
}

template <int EL, int OUT>
hipError_t launch_combine_shapes(int shape, bool packed, const GemmProblem& p, int max_tiles, hipStream_t stream) {
  if (shape == kShapeTile256)
    return packed ? launch_one<EL, OUT, false, kShapeTile256, true, true>(p, max_tiles, stream)
                  : launch_one<EL, OUT, false, kShapeTile256, false, true>(p, max_tiles, stream);
  return packed ? launch_one<EL, OUT, false, kShapeStream32, true, true>(p, max_tiles, stream)
                : launch_one<EL, OUT, false, kShapeStream32, false, true>(p, max_tiles, stream);
}

template <int EL, int OUT, bool SWIGLU, bool PACKED>
hipError_t launch_layout(int shape, const GemmProblem& p, int max_tiles, hipStream_t stream) {
  switch (shape) {
    case kShapeStream16: return launch_one<EL, OUT, SWIGLU, kShapeStream16, PACKED>(p, max_tiles, stream);
    case kShapeStream32: return launch_one<EL, OUT, SWIGLU, kShapeStream32, PACKED>(p, max_tiles, stream);
    default: return launch_one<EL, OUT, SWIGLU, kShapeTile256, PACKED>(p, max_tiles, stream);
  }
}

template <int EL, int OUT, bool SWIGLU>
hipError_t launch_shape(int shape, bool packed, const GemmProblem& p, int max_tiles, hipStream_t stream) {
  return packed ? launch_layout<EL, OUT, SWIGLU, true>(shape, p, max_tiles, stream)
                : launch_layout<EL, OUT, SWIGLU, false>(shape, p, max_tiles, stream);
}

}  // namespace

hipError_t launch_gemm(int el, int out_el, bool swiglu, int shape, bool packed, const GemmProblem& p, int max_tiles,
                       hipStream_t stream) {
#define MOE_GEMM(E_, O_, S_) \
  return launch_shape<E_, O_, S_>(shape, packed, p, max_tiles, stream)
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

hipError_t launch_gemm_combine(int el, int out_el, int shape, bool packed, const GemmProblem& p, int max_tiles,
                               hipStream_t stream) {
  if (!p.comb_rows || !p.comb_packed || !p.comb_inv || p.offsets || p.perm || p.k_splits != 1)
    return hipErrorInvalidValue;
  if (shape != kShapeTile256 && shape != kShapeStream32) return hipErrorInvalidValue;
  if (el == EL_F32 && out_el == EL_F32) return launch_combine_shapes<EL_F32, EL_F32>(shape, packed, p, max_tiles, stream);
  if (el == EL_BF16 && out_el == EL_BF16)
    return launch_combine_shapes<EL_BF16, EL_BF16>(shape, packed, p, max_tiles, stream);
  if (el == EL_BF16 && out_el == EL_F32)
    return launch_combine_shapes<EL_BF16, EL_F32>(shape, packed, p, max_tiles, stream);
  return hipErrorInvalidValue;
}

}  // namespace moe
