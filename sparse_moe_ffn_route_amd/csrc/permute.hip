// Grouping (token, slot) pairs by expert, its inverse map, row gathers and the
// per-row E4M3 quantiser.
//
// Source: the grouped GEMMs and the "unpermutation + local reduction" of
// "Systems Engineering Playbook: Qwen 3.5 MoE on Ironwood TPU" (table "Three
// High-Leverage Optimizations") need the rows of each expert contiguous; under
// expert parallelism only the device's own expert slice is grouped (section
// "Fusing Three Collectives Into Two").
//
// Deterministic without atomics deciding positions: lanes holding the same expert find
// each other with one ballot per bit of the expert id and rank themselves by lane
// order; the lowest lane advances that expert's running count.  The row of a pair is
// (rows of lower experts) + (earlier pairs of the same expert), i.e. experts ascending
// and (t, j) ascending inside an expert.
//   * up to 8192 pairs (decode sizes): one 1024-thread workgroup does everything;
//   * beyond: rank within 1024-pair units (one wave each), one-workgroup scan over
//     experts, then one thread per pair places it.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kWavesPerBlock = 4;

constexpr int kUnitSteps = kPermUnit / kWave;  // 64-pair steps of one unit (16)
constexpr int kScanLds = 16384;                // histogram entries the scan stages in LDS (64 KB)

// Local expert of pair i of the token-major list, -1 if the expert is not local.
__device__ __forceinline__ int local_expert(const int32_t* packed, int i, int k, int e_begin, int n_local) {
  const int t = i / k;
  const int e = packed[static_cast<size_t>(t) * 2 * k + (i - t * k)] - e_begin;
  return (e >= 0 && e < n_local) ? e : -1;
}

// Local expert of pair i as local_expert(), and whether its id lies outside [0, E) (a
// corrupt or foreign blob: such a pair is skipped and counted).
__device__ __forceinline__ int local_expert_checked(const int32_t* packed, int i, int k, int e_begin, int n_local,
                                                    int E, bool& bad) {
  const int t = i / k;
  const int id = packed[static_cast<size_t>(t) * 2 * k + (i - t * k)];
  bad = id < 0 || id >= E;
  const int e = id - e_begin;
  return (e >= 0 && e < n_local) ? e : -1;
}

// Per-row E4M3 quantisation of row r by one wave (defined with quant_rows_kernel).
template <int IN>
__device__ __forceinline__ void quant_row(const void* __restrict__ src, int r, int cols, int lane,
                                          uint8_t* __restrict__ dst, float* __restrict__ scale);

// Stage 1 of the multi-workgroup grouping: one wave per unit of kPermUnit consecutive
// pairs.  The wave loads all its pairs first (one memory latency), then walks them 64
// at a time: lanes holding the same expert find each other with one ballot per id bit,
// rank themselves by lane order, and the lowest lane advances that expert's running
// count in LDS.  Output: each local pair's rank inside its unit, hist[unit][e], and
// bad[unit], the unit's pairs whose id lies outside [0, E).
// Workgroups from rank_blocks on quantise the bf16 token rows qsrc [qrows][qcols] to
// E4M3 (one wave per row): that needs nothing from the grouping, so it runs beside the
// ranking instead of after the grouping.
__global__ __launch_bounds__(256) void perm_rank_kernel(const int32_t* __restrict__ packed, int n_pairs, int k,
                                                        int e_begin, int n_local, int E, int n_bits, int n_units,
                                                        int32_t* __restrict__ rank, int32_t* __restrict__ hist,
                                                        int32_t* __restrict__ bad, int rank_blocks,
                                                        const void* __restrict__ qsrc, int qrows, int qcols,
                                                        uint8_t* __restrict__ qdst, float* __restrict__ qscale) {
  __shared__ int32_t run[kWavesPerBlock][kMaxLocalExperts];
  const int w = threadIdx.x / kWave, lane = lane_id();
  if (static_cast<int>(blockIdx.x) >= rank_blocks) {
    const int r = (static_cast<int>(blockIdx.x) - rank_blocks) * kWavesPerBlock + w;
    if (r < qrows) quant_row<EL_BF16>(qsrc, r, qcols, lane, qdst, qscale);
    return;
  }
  const int u = blockIdx.x * kWavesPerBlock + w;
  if (u >= n_units) return;  // whole wave leaves together; waves use disjoint LDS rows
  const int base_i = u * kPermUnit;
  int pe[kUnitSteps];
  int n_bad = 0;  // wave-uniform
#pragma unroll
  for (int s = 0; s < kUnitSteps; ++s) {
    const int i = base_i + s * kWave + lane;
    bool b = false;
    pe[s] = i < n_pairs ? local_expert_checked(packed, i, k, e_begin, n_local, E, b) : -1;
    n_bad += __popcll(__ballot(b));
  }
  if (lane == 0) bad[u] = n_bad;
  for (int e = lane; e < n_local; e += kWave) run[w][e] = 0;
  __builtin_amdgcn_wave_barrier();
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int s = 0; s < kUnitSteps; ++s) {
    const int e = pe[s];
    const bool local = e >= 0;
    uint64_t same = __ballot(local);
    for (int b = 0; b < n_bits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t m = __ballot(local && bit);
      same &= bit ? m : ~m;
    }
    const int r = __popcll(same & below);
    if (local) rank[base_i + s * kWave + lane] = run[w][e] + r;
    __builtin_amdgcn_wave_barrier();  // every lane has read its count before the leaders advance it
    if (local && r == 0) run[w][e] += __popcll(same);
    __builtin_amdgcn_wave_barrier();
  }
  for (int e = lane; e < n_local; e += kWave) hist[static_cast<size_t>(u) * n_local + e] = run[w][e];
}

// Stage 2: one workgroup, thread e owns expert e (n_local <= 1024).  Expert totals and
// M-tile counts are scanned over experts; hist[unit][e] becomes base[unit][e], the first
// grouped row of expert e coming from that unit.  Each pass over units reads one
// contiguous row of n_local counts across the workgroup.
// It also adds the units' counts of out-of-range ids into *err_word.
__global__ __launch_bounds__(1024) void perm_scan_kernel(const int32_t* __restrict__ hist, int n_local,
                                                         int n_units, int bm0, int bm1, int32_t* __restrict__ base,
                                                         int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ prefix0,
                                                         int32_t* __restrict__ prefix1,
                                                         const int32_t* __restrict__ bad,
                                                         int32_t* __restrict__ err_word) {
  __shared__ int32_t sc[3][1024];
  __shared__ int32_t sbad[1024 / kWave];
  __shared__ int32_t sh[kScanLds];  // the whole histogram, when it fits
  const int e = threadIdx.x;
  {
    int nb = 0;
    for (int u = e; u < n_units; u += 1024) nb += bad[u];
    nb = wave_sum_int(nb);
    if (lane_id() == 0) sbad[e / kWave] = nb;
  }
  // A histogram that fits in LDS is loaded by the whole workgroup in one coalesced sweep
  // (one memory latency), rather than unit by unit by each expert's thread.
  const int n_hist = n_units * n_local;
  const bool in_lds = n_hist <= kScanLds;
  if (in_lds) {
    for (int i = e; i < n_hist; i += 1024) sh[i] = hist[i];
    __syncthreads();
  }
  const int32_t* hsrc = in_lds ? sh : hist;
  int tot = 0;
  if (e < n_local) {
#pragma unroll 8
    for (int u = 0; u < n_units; ++u) tot += hsrc[static_cast<size_t>(u) * n_local + e];
  }
  sc[0][e] = tot;
  sc[1][e] = (tot + bm0 - 1) / bm0;
  sc[2][e] = (tot + bm1 - 1) / bm1;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    int a = 0, b = 0, c = 0;
    if (e >= o) {
      a = sc[0][e - o];
      b = sc[1][e - o];
      c = sc[2][e - o];
    }
    __syncthreads();
    sc[0][e] += a;
    sc[1][e] += b;
    sc[2][e] += c;
    __syncthreads();
  }
  if (e < n_local) {
    int run = sc[0][e] - tot;
    counts[e] = tot;
    offsets[e] = run;
    prefix0[e + 1] = sc[1][e];
    prefix1[e + 1] = sc[2][e];
#pragma unroll 8
    for (int u = 0; u < n_units; ++u) {
      const size_t at = static_cast<size_t>(u) * n_local + e;
      const int c = hsrc[at];
      base[at] = run;
      run += c;
    }
  }
  if (e == 0) {
    offsets[n_local] = sc[0][1023];
    prefix0[0] = 0;
    prefix1[0] = 0;
    int nb = 0;
    for (int w = 0; w < 1024 / kWave; ++w) nb += sbad[w];  // sbad is complete: barriers above
    *err_word = nb;
  }
}

// Stage 3: one thread per pair: row = base[e][unit] + rank inside the unit.
__global__ __launch_bounds__(256) void perm_place_kernel(const int32_t* __restrict__ packed, int n_pairs, int k,
                                                         int e_begin, int n_local, int n_units,
                                                         const int32_t* __restrict__ base,
                                                         const int32_t* __restrict__ rank,
                                                         int32_t* __restrict__ perm_token,
                                                         int32_t* __restrict__ inv_pos) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_pairs) return;
  const int e = local_expert(packed, i, k, e_begin, n_local);
  int pos = -1;
  if (e >= 0) {
    pos = base[static_cast<size_t>(i / kPermUnit) * n_local + e] + rank[i];
    perm_token[pos] = i / k;
  }
  inv_pos[i] = pos;
}

// Whole grouping in one 1024-thread workgroup (used up to 16 * 64 * 8 pairs):
// 16 waves each own one contiguous range of pairs.  Every lane first loads all of its
// pairs into registers in one batch (one memory latency instead of one per 64 pairs),
// packed as (token << 11) | (local expert + 1), 0 in the low bits for a non-local
// expert.  The per-wave histograms, the expert-major scan (with the M-tile prefixes of
// both GEMMs) and the ballot-ranked scatter then run from registers and LDS, in one
// launch.
constexpr int kFusedWaves = 16;

// MAXSTEPS: compile-time bound on the 64-pair steps of one wave (the register array of
// preloaded pairs); a small instance keeps the decode-sized launch's code short.
template <int MAXSTEPS>
__global__ __launch_bounds__(1024) void perm_fused_kernel(const int32_t* __restrict__ packed, int n_pairs, int k,
                                                          int e_begin, int n_local, int n_bits, int bm0, int bm1,
                                                          int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ perm_token,
                                                          int32_t* __restrict__ inv_pos, int32_t* __restrict__ prefix0,
                                                          int32_t* __restrict__ prefix1, int E,
                                                          int32_t* __restrict__ err_word) {
  __shared__ int32_t hist[kFusedWaves][kMaxLocalExperts];
  __shared__ int32_t sc[3][1024];
  __shared__ int32_t sbad[kFusedWaves];
  const int tid = threadIdx.x, w = tid / kWave, lane = lane_id();
  const int per_wave = ((n_pairs + kFusedWaves * kWave - 1) / (kFusedWaves * kWave)) * kWave;
  const int lo = min(n_pairs, w * per_wave), hi = min(n_pairs, lo + per_wave);
  const int nsteps = (hi - lo + kWave - 1) / kWave;

  int pv[MAXSTEPS];  // -1: past the end; else (t << 11) | (local expert + 1 or 0)
  int n_bad = 0;     // pairs of this wave whose id lies outside [0, E) (wave-uniform)
#pragma unroll
  for (int s = 0; s < MAXSTEPS; ++s) {
    pv[s] = -1;
    if (s < nsteps) {
      const int i = lo + s * kWave + lane;
      bool b = false;
      if (i < hi) {
        const int t = i / k;
        const int id = packed[static_cast<size_t>(t) * 2 * k + (i - t * k)];
        b = id < 0 || id >= E;
        const int e = id - e_begin;
        pv[s] = (t << 11) | ((e >= 0 && e < n_local) ? e + 1 : 0);
      }
      n_bad += __popcll(__ballot(b));
    }
  }
  if (lane == 0) sbad[w] = n_bad;

  for (int e = lane; e < n_local; e += kWave) hist[w][e] = 0;
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int s = 0; s < MAXSTEPS; ++s) {
    if (s < nsteps) {
      const int e = (pv[s] & 2047) - 1;
      if (pv[s] >= 0 && e >= 0) atomicAdd(&hist[w][e], 1);
    }
  }
  __syncthreads();

  // expert e = tid: total rows and M-tiles; inclusive scans over experts
  int tot = 0;
  if (tid < n_local)
    for (int v = 0; v < kFusedWaves; ++v) tot += hist[v][tid];
  const int t0 = (tot + bm0 - 1) / bm0, t1 = (tot + bm1 - 1) / bm1;
  sc[0][tid] = tot;
  sc[1][tid] = t0;
  sc[2][tid] = t1;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    int a = 0, b = 0, c = 0;
    if (tid >= o) {
      a = sc[0][tid - o];
      b = sc[1][tid - o];
      c = sc[2][tid - o];
    }
    __syncthreads();
    sc[0][tid] += a;
    sc[1][tid] += b;
    sc[2][tid] += c;
    __syncthreads();
  }
  if (tid < n_local) {
    const int ex = sc[0][tid] - tot;
    counts[tid] = tot;
    offsets[tid] = ex;
    prefix0[tid + 1] = sc[1][tid];
    prefix1[tid + 1] = sc[2][tid];
    int run = ex;  // column tid becomes each wave's first row of expert tid
    for (int v = 0; v < kFusedWaves; ++v) {
      const int c = hist[v][tid];
      hist[v][tid] = run;
      run += c;
    }
  }
  if (tid == 0) {
    offsets[n_local] = sc[0][1023];
    prefix0[0] = 0;
    prefix1[0] = 0;
    int nb = 0;
    for (int v = 0; v < kFusedWaves; ++v) nb += sbad[v];  // written before the first barrier
    *err_word = nb;
  }
  __syncthreads();

  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int s = 0; s < MAXSTEPS; ++s) {
    if (s < nsteps) {
      const bool valid = pv[s] >= 0;
      const int e = valid ? (pv[s] & 2047) - 1 : -1;
      const bool local = e >= 0;
      uint64_t same = __ballot(local);
      for (int b = 0; b < n_bits; ++b) {
        const bool bit = (e >> b) & 1;
        const uint64_t m = __ballot(local && bit);
        same &= bit ? m : ~m;
      }
      int pos = -1;
      const int rank = __popcll(same & below);
      if (local) {
        pos = hist[w][e] + rank;
        perm_token[pos] = pv[s] >> 11;
      }
      __builtin_amdgcn_wave_barrier();  // every lane has read its base before the leaders advance it
      if (local && rank == 0) hist[w][e] += __popcll(same);
      __builtin_amdgcn_wave_barrier();
      if (valid) inv_pos[lo + s * kWave + lane] = pos;
    }
  }
}

// Row gather: dst[r] = src[perm_token[r]] for r < offsets[n_local]; bytes per row
// must be a multiple of 16.  One 256-thread block per row.
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint8_t* __restrict__ src,
                                                          const float* __restrict__ src_scale,
                                                          const int32_t* __restrict__ perm_token,
                                                          const int32_t* __restrict__ n_rows_dev,
                                                          int row_bytes, uint8_t* __restrict__ dst,
                                                          float* __restrict__ dst_scale) {
  const int r = blockIdx.x;
  if (r >= *n_rows_dev) return;
  const int t = perm_token[r];
  const uint4* s = reinterpret_cast<const uint4*>(src + static_cast<size_t>(t) * row_bytes);
  uint4* d = reinterpret_cast<uint4*>(dst + static_cast<size_t>(r) * row_bytes);
  for (int c = threadIdx.x; c < row_bytes / 16; c += blockDim.x) d[c] = s[c];
  if (dst_scale && threadIdx.x == 0) dst_scale[r] = src_scale[t];
}

// Per-row E4M3 quantisation: s = amax / 448 (1 for an all-zero row), q = E4M3(v / s).
// One wave per row; rows counted by *n_rows_dev when given (device-side row count).
// Rows of at most 4096 columns are read once: each lane issues the loads of all its
// 8-column pieces together (2, 4 or 8 of them, by row width) and keeps them in
// registers for both the amax and the quantisation pass; wider rows are read twice.
// One row held in registers: P 8-column pieces per lane (cols <= 512 * P).
template <int IN, int P>
__device__ __forceinline__ void quant_row_in_regs(const void* __restrict__ src, int r, int cols, int lane,
                                                  uint8_t* __restrict__ dst, float* __restrict__ scale) {
  // Branch-free loads: a piece past the row end re-reads the row's last piece and
  // is masked out of the amax and not stored.
  float v[P][8];
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const int c = min((i * kWave + lane) * 8, cols - 8);
    if (IN == EL_BF16) {
      const uint4 p =
          *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(src) + static_cast<size_t>(r) * cols + c);
      const uint32_t wds[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[i][2 * q] = bf16_bits_to_f32(wds[q] & 0xFFFFu);
        v[i][2 * q + 1] = bf16_bits_to_f32(wds[q] >> 16);
      }
    } else {
      const float4* p =
          reinterpret_cast<const float4*>(static_cast<const float*>(src) + static_cast<size_t>(r) * cols + c);
      const float4 a = p[0], b = p[1];
      v[i][0] = a.x; v[i][1] = a.y; v[i][2] = a.z; v[i][3] = a.w;
      v[i][4] = b.x; v[i][5] = b.y; v[i][6] = b.z; v[i][7] = b.w;
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const bool in_row = (i * kWave + lane) * 8 < cols;
#pragma unroll
    for (int q = 0; q < 8; ++q) amax = fmaxf(amax, in_row ? fabsf(v[i][q]) : 0.0f);
  }
  amax = wave_max(amax);
  const float s = (amax == 0.0f) ? 1.0f : amax / 448.0f;
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const int c = (i * kWave + lane) * 8;
    if (c >= cols) continue;
    uint32_t packed4[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const float a0 = fminf(fmaxf(v[i][4 * q + 0] / s, -448.0f), 448.0f);
      const float a1 = fminf(fmaxf(v[i][4 * q + 1] / s, -448.0f), 448.0f);
      const float a2 = fminf(fmaxf(v[i][4 * q + 2] / s, -448.0f), 448.0f);
      const float a3 = fminf(fmaxf(v[i][4 * q + 3] / s, -448.0f), 448.0f);
      packed4[q] = f32x2_to_e4m3x2(a0, a1) | (f32x2_to_e4m3x2(a2, a3) << 16);
    }
    *reinterpret_cast<uint2*>(dst + static_cast<size_t>(r) * cols + c) = make_uint2(packed4[0], packed4[1]);
  }
  if (lane == 0) scale[r] = s;
}

template <int IN>
__device__ __forceinline__ void quant_row(const void* __restrict__ src, int r, int cols, int lane,
                                          uint8_t* __restrict__ dst, float* __restrict__ scale) {
  if (cols <= kWave * 8 * 2) return quant_row_in_regs<IN, 2>(src, r, cols, lane, dst, scale);
  if (cols <= kWave * 8 * 4) return quant_row_in_regs<IN, 4>(src, r, cols, lane, dst, scale);
  if (cols <= kWave * 8 * 8) return quant_row_in_regs<IN, 8>(src, r, cols, lane, dst, scale);
  // each lane handles 8 consecutive values per step
  float amax = 0.0f;
  for (int c = lane * 8; c < cols; c += kWave * 8) {
    float v[8];
    if (IN == EL_BF16) {
      const uint4 p = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(src) + static_cast<size_t>(r) * cols + c);
      const uint32_t wds[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[2 * q] = bf16_bits_to_f32(wds[q] & 0xFFFFu);
        v[2 * q + 1] = bf16_bits_to_f32(wds[q] >> 16);
      }
    } else {
      const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(src) + static_cast<size_t>(r) * cols + c);
      const float4 a = p[0], b = p[1];
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) amax = fmaxf(amax, fabsf(v[q]));
  }
  amax = wave_max(amax);
  const float s = (amax == 0.0f) ? 1.0f : amax / 448.0f;
  for (int c = lane * 8; c < cols; c += kWave * 8) {
    float v[8];
    if (IN == EL_BF16) {
      const uint4 p = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(src) + static_cast<size_t>(r) * cols + c);
      const uint32_t wds[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[2 * q] = bf16_bits_to_f32(wds[q] & 0xFFFFu);
        v[2 * q + 1] = bf16_bits_to_f32(wds[q] >> 16);
      }
    } else {
      const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(src) + static_cast<size_t>(r) * cols + c);
      const float4 a = p[0], b = p[1];
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
    uint32_t packed4[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      float a0 = fminf(fmaxf(v[4 * q + 0] / s, -448.0f), 448.0f);
      float a1 = fminf(fmaxf(v[4 * q + 1] / s, -448.0f), 448.0f);
      float a2 = fminf(fmaxf(v[4 * q + 2] / s, -448.0f), 448.0f);
      float a3 = fminf(fmaxf(v[4 * q + 3] / s, -448.0f), 448.0f);
      packed4[q] = f32x2_to_e4m3x2(a0, a1) | (f32x2_to_e4m3x2(a2, a3) << 16);
    }
    *reinterpret_cast<uint2*>(dst + static_cast<size_t>(r) * cols + c) = make_uint2(packed4[0], packed4[1]);
  }
  if (lane == 0) scale[r] = s;
}

// skip_inv: NULL, or inv_pos [rows][skip_k]: a row whose k slots are all non-local
// (inv_pos < 0) is never read by the grouped GEMMs and is left unwritten.
template <int IN>
__global__ __launch_bounds__(256) void quant_rows_kernel(const void* __restrict__ src, int rows,
                                                         const int32_t* __restrict__ n_rows_dev, int cols,
                                                         uint8_t* __restrict__ dst, float* __restrict__ scale,
                                                         const int32_t* __restrict__ skip_inv, int skip_k) {
  const int r = blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
  const int lane = lane_id();
  const int n = n_rows_dev ? *n_rows_dev : rows;
  if (r >= n) return;
  if (skip_inv) {
    const bool used = lane < skip_k && skip_inv[static_cast<size_t>(r) * skip_k + lane] >= 0;
    if (__ballot(used) == 0) return;  // wave-uniform
  }
  quant_row<IN>(src, r, cols, lane, dst, scale);
}

// Tile schedule: prefix[g] = sum over groups g' < g of ceil(rows_g' / bm), for two
// tile heights at once.  One workgroup of 1024 threads (n_groups <= 1024).
__global__ __launch_bounds__(1024) void tile_prefix_kernel(const int32_t* __restrict__ offsets, int n_groups,
                                                           int bm0, int bm1, int32_t* __restrict__ prefix0,
                                                           int32_t* __restrict__ prefix1) {
  __shared__ int32_t p0[1024], p1[1024];
  const int g = threadIdx.x;
  int c0 = 0, c1 = 0;
  if (g < n_groups) {
    const int rows = offsets[g + 1] - offsets[g];
    c0 = (rows + bm0 - 1) / bm0;
    c1 = (rows + bm1 - 1) / bm1;
  }
  p0[g] = c0;
  p1[g] = c1;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int v0 = g >= o ? p0[g - o] : 0;
    const int v1 = g >= o ? p1[g - o] : 0;
    __syncthreads();
    p0[g] += v0;
    p1[g] += v1;
    __syncthreads();
  }
  if (g < n_groups) {
    prefix0[g + 1] = p0[g];
    prefix1[g + 1] = p1[g];
  }
  if (g == 0) {
    prefix0[0] = 0;
    prefix1[0] = 0;
  }
}

}  // namespace

hipError_t launch_permute(const int32_t* packed, int T, int k, int E, int e_begin, int n_local, int32_t* hist,
                          int32_t* base, int32_t* rank, int32_t* bad, int32_t* counts, int32_t* offsets,
                          int32_t* perm_token, int32_t* inv_pos, int bm0, int bm1, int32_t* prefix0,
                          int32_t* prefix1, int32_t* err_word, hipStream_t stream, const void* xq_src, int xq_cols,
                          void* xq_dst, float* xq_scale) {
  const int n_pairs = T * k;
  int n_bits = 1;
  while ((1 << n_bits) < n_local) ++n_bits;
  if (n_pairs <= kFusedWaves * kWave * 8) {
    hipLaunchKernelGGL(perm_fused_kernel<8>, dim3(1), dim3(1024), 0, stream, packed, n_pairs, k, e_begin, n_local,
                       n_bits, bm0, bm1, counts, offsets, perm_token, inv_pos, prefix0, prefix1, E, err_word);
    if (!xq_src) return hipGetLastError();
    // tokens without a local slot (other devices' experts only) are not quantised
    return launch_quant_rows(EL_BF16, xq_src, T, nullptr, xq_cols, xq_dst, xq_scale, stream, inv_pos, k);
  }
  const int n_units = perm_units(T, k);
  const int blocks = (n_units + kWavesPerBlock - 1) / kWavesPerBlock;
  const int q_blocks = xq_src ? (T + kWavesPerBlock - 1) / kWavesPerBlock : 0;
  hipLaunchKernelGGL(perm_rank_kernel, dim3(blocks + q_blocks), dim3(256), 0, stream, packed, n_pairs, k, e_begin,
                     n_local, E, n_bits, n_units, rank, hist, bad, blocks, xq_src, xq_src ? T : 0, xq_cols,
                     static_cast<uint8_t*>(xq_dst), xq_scale);
  hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(1024), 0, stream, hist, n_local, n_units, bm0, bm1, base,
                     counts, offsets, prefix0, prefix1, bad, err_word);
  hipLaunchKernelGGL(perm_place_kernel, dim3((n_pairs + 255) / 256), dim3(256), 0, stream, packed, n_pairs, k,
                     e_begin, n_local, n_units, base, rank, perm_token, inv_pos);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void* src, const float* src_scale, const int32_t* perm_token,
                              const int32_t* n_rows_dev, int max_rows, int row_bytes, void* dst, float* dst_scale,
                              hipStream_t stream) {
  if (max_rows == 0) return hipSuccess;
  hipLaunchKernelGGL(gather_rows_kernel, dim3(max_rows), dim3(256), 0, stream,
                     static_cast<const uint8_t*>(src), src_scale, perm_token, n_rows_dev, row_bytes,
                     static_cast<uint8_t*>(dst), dst_scale);
  return hipGetLastError();
}

hipError_t launch_quant_rows(int in_el, const void* src, int rows, const int32_t* n_rows_dev, int cols, void* dst,
                             float* scale, hipStream_t stream, const int32_t* skip_inv, int skip_k) {
  if (rows == 0) return hipSuccess;
  dim3 grid((rows + kWavesPerBlock - 1) / kWavesPerBlock);
  if (in_el == EL_BF16)
    hipLaunchKernelGGL(quant_rows_kernel<EL_BF16>, grid, dim3(256), 0, stream, src, rows, n_rows_dev, cols,
                       static_cast<uint8_t*>(dst), scale, skip_inv, skip_k);
  else
    hipLaunchKernelGGL(quant_rows_kernel<EL_F32>, grid, dim3(256), 0, stream, src, rows, n_rows_dev, cols,
                       static_cast<uint8_t*>(dst), scale, skip_inv, skip_k);
  return hipGetLastError();
}

hipError_t launch_tile_prefix(const int32_t* offsets, int n_groups, int bm0, int bm1, int32_t* prefix0,
                              int32_t* prefix1, hipStream_t stream) {
  hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(1024), 0, stream, offsets, n_groups, bm0, bm1, prefix0,
                     prefix1);
  return hipGetLastError();
}

}  // namespace moe
