// Dynamic partial-KV update for CDNA4 (gfx950): key scoring, exact top-budget
// selection and the gather of the partial cache.
//
// What is computed (TokenSwift summary §3.3 "Dynamic KV Cache Management"):
// per KV head g, the grouped importance score of every committed row
//   sigma[g][j] = sum_{h in group g} sum_t q[h][t] . k[g][j] = qbar_g . k[g][j]
// (the sum over queries moves inside the dot product: one K pass), the B'
// best candidates in (score desc, row asc) order, and the partial cache
// sink U selected U recent.
//
// Kernels (one stream, in order):
//   1. prologue  grid Hkv:  qbar_g in fp32, clear the per-head histogram.
//   2. score     grid (chunks, Hkv): one HBM pass over K. 16 lanes x 16 B per
//                row (d=128), lane-local FMAs then a 16-lane reduction; the
//                block also histograms the top 12 bits of each candidate's
//                order-preserving key and adds its non-empty bins to the
//                head's global histogram.
//   3. select    grid Hkv, 1024 threads: the top-12-bit bin holding the B'-th
//                key comes from the histogram; two more radix passes (10 + 10
//                bits) over the L2-resident scores fix the exact cut key;
//                a block-wide ordered scan then emits the rows above the cut
//                plus the earliest ties, ascending.
//   4. gather    grid (row chunks, Hkv): copy sink, selected and recent rows of
//                K and V into the partial cache.
#include "ts_internal.h"

#include <cmath>

namespace ts {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int HIST1_BITS = 12;
constexpr int HIST1 = 1 << HIST1_BITS;  // bins of the first radix digit
constexpr int SEL_THREADS = 1024;

// Order-preserving map from float to uint32 (larger float -> larger key).
__device__ inline unsigned int f2key(float f) {
  const unsigned int u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ inline float bf16_lo(unsigned int w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(unsigned int w) { return __uint_as_float(w & 0xffff0000u); }

// Lanes below the caller's in the wave.
__device__ inline unsigned long long lanemask_lt() {
  return (1ull << (threadIdx.x & 63)) - 1ull;
}
__device__ inline unsigned int popc64(unsigned long long x) { return (unsigned int)__popcll(x); }

// qbar_g[c] = sum over the group's query rows (G heads x T queries) in fp32.
// Each thread sums 8 channels of every 256/(D/8)-th row, then an LDS
// reduction over the row slots (fixed order: deterministic).
template <int D>
__global__ __launch_bounds__(256) void select_prologue_kernel(const SelectParams p, unsigned int* hist) {
  constexpr int LPR = D / 8;          // lanes per row
  constexpr int RS = 256 / LPR;       // row slots
  __shared__ float part[RS][D];
  const int g = blockIdx.x;
  const int tid = threadIdx.x;
  const int cg = tid % LPR, rs = tid / LPR;
  const int rows = (p.Hq / p.Hkv) * p.T;
  const uint16_t* qg = p.q + (int64_t)g * rows * D + cg * 8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int r = rs; r < rows; r += RS) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(qg + (int64_t)r * D);
    acc[0] += bf16_lo(w.x); acc[1] += bf16_hi(w.x);
    acc[2] += bf16_lo(w.y); acc[3] += bf16_hi(w.y);
    acc[4] += bf16_lo(w.z); acc[5] += bf16_hi(w.z);
    acc[6] += bf16_lo(w.w); acc[7] += bf16_hi(w.w);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[rs][cg * 8 + e] = acc[e];
  for (int b = tid; b < HIST1; b += 256) hist[g * HIST1 + b] = 0u;
  __syncthreads();
  if (tid < D) {
    float t = 0.f;
    for (int q = 0; q < RS; ++q) t += part[q][tid];
    p.qbar[g * D + tid] = t;
  }
}

// LPR lanes per row, each holding 8 channels; a wave covers 64/LPR rows.
template <int D>
__global__ __launch_bounds__(256) void select_score_kernel(const SelectParams p, unsigned int* ghist, int rows_per_block) {
  constexpr int LPR = D / 8;
  constexpr int RPW = 64 / LPR;   // rows per wave per step
  constexpr int UNROLL = 4;
  __shared__ unsigned int lhist[HIST1];
  const int g = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int sub = lane % LPR;
  const int rsub = lane / LPR;
  for (int b = tid; b < HIST1; b += 256) lhist[b] = 0u;

  float qb[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) qb[e] = p.qbar[g * D + sub * 8 + e];
  __syncthreads();

  const int r0 = blockIdx.x * rows_per_block;
  const int r1 = min(r0 + rows_per_block, p.n_ctx);
  const uint16_t* kg = p.k + (int64_t)g * p.s_head + sub * 8;
  float* sc = p.scores + (int64_t)g * p.n_ctx;
  // each wave walks rows r0 + wave*RPW*UNROLL + ..., UNROLL groups of RPW rows in flight
  for (int base = r0 + wave * RPW * UNROLL; base < r1; base += 4 * RPW * UNROLL) {
    u32x4 w[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int j = base + u * RPW + rsub;
      w[u] = u32x4{0u, 0u, 0u, 0u};
      if (j < r1) w[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kg + (int64_t)j * p.s_pos));
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      float acc = 0.f;
      acc = fmaf(qb[0], bf16_lo(w[u].x), acc);
      acc = fmaf(qb[1], bf16_hi(w[u].x), acc);
      acc = fmaf(qb[2], bf16_lo(w[u].y), acc);
      acc = fmaf(qb[3], bf16_hi(w[u].y), acc);
      acc = fmaf(qb[4], bf16_lo(w[u].z), acc);
      acc = fmaf(qb[5], bf16_hi(w[u].z), acc);
      acc = fmaf(qb[6], bf16_lo(w[u].w), acc);
      acc = fmaf(qb[7], bf16_hi(w[u].w), acc);
#pragma unroll
      for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
      const int j = base + u * RPW + rsub;
      if (sub == 0 && j < r1) {
        sc[j] = acc;
        if (j >= p.cand_lo && j < p.cand_hi) atomicAdd(&lhist[f2key(acc) >> (32 - HIST1_BITS)], 1u);
      }
    }
  }
  __syncthreads();
  for (int b = tid; b < HIST1; b += 256) {
    const unsigned int c = lhist[b];
    if (c) atomicAdd(&ghist[g * HIST1 + b], c);
  }
}

// Block-wide exclusive scan over SEL_THREADS threads; returns the prefix and
// the total. `tmp` holds one slot per wave.
__device__ inline unsigned int block_exclusive_scan(unsigned int x, unsigned int* tmp, unsigned int* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  unsigned int incl = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const unsigned int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) tmp[wave] = incl;
  __syncthreads();
  unsigned int wave_prefix = 0, tot = 0;
  for (int w = 0; w < SEL_THREADS / 64; ++w) {
    const unsigned int t = tmp[w];
    if (w < wave) wave_prefix += t;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return wave_prefix + incl - x;
}

// Find, scanning bins from the top, the bin holding the k-th largest key
// (k >= 1). hist has nbins entries in LDS; sets *bin and *above (the count in
// higher bins). Each thread owns nbins / SEL_THREADS consecutive bins.
__device__ inline void find_bin(const unsigned int* hist, int nbins, unsigned int k, unsigned int* tmp, int* bin_out,
                                unsigned int* above_out) {
  const int per = nbins / SEL_THREADS;
  // thread t covers the t-th group of bins counted from the top
  const int hi_bin = nbins - 1 - threadIdx.x * per;
  unsigned int s = 0;
  for (int i = 0; i < per; ++i) s += hist[hi_bin - i];
  unsigned int total;
  const unsigned int before = block_exclusive_scan(s, tmp, &total);
  if (before < k && k <= before + s) {
    unsigned int acc = before;
    for (int i = 0; i < per; ++i) {
      const unsigned int c = hist[hi_bin - i];
      if (acc + c >= k) {
        *bin_out = hi_bin - i;
        *above_out = acc;
        break;
      }
      acc += c;
    }
  }
  __syncthreads();
}

constexpr int CAND_CAP = 16384;  // candidate keys of the cut bin held in LDS
constexpr int UNR = 32;          // wave steps whose loads are in flight together (~128 KB per CU)

// Ordered pass of one wave over rows [s0, s1), 64 rows per step in ascending
// order, UNR steps' loads in flight; f(j, valid, key) is called by all lanes.
template <typename F>
__device__ inline void wave_pass_keys(const float* sc, int s0, int s1, F&& f) {
  const int lane = threadIdx.x & 63;
  for (int b0 = s0; b0 < s1; b0 += UNR * 64) {
    float v[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int j = b0 + u * 64 + lane;
      v[u] = j < s1 ? sc[j] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int j = b0 + u * 64 + lane;
      if (b0 + u * 64 < s1) f(j, j < s1, f2key(v[u]));
    }
  }
}

__global__ __launch_bounds__(SEL_THREADS) void select_topb_kernel(const SelectParams p, const unsigned int* ghist) {
  __shared__ unsigned int hist[HIST1];
  __shared__ unsigned int cand[CAND_CAP];
  __shared__ unsigned int tmp[SEL_THREADS / 64];
  __shared__ unsigned int wave_gt[SEL_THREADS / 64], wave_tie[SEL_THREADS / 64];
  __shared__ int s_bin;
  __shared__ unsigned int s_above, s_ncand;
  const int g = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  int32_t* out = p.sel_idx + (int64_t)g * p.budget;
  const unsigned int k = (unsigned int)p.b_eff;
  for (int i = k + tid; i < p.budget; i += SEL_THREADS) out[i] = -1;
  if (k == 0) return;
  const float* sc = p.scores + (int64_t)g * p.n_ctx;
  const int lo = p.cand_lo, hi = p.cand_hi;

  // digit 1 (top 12 key bits): the histogram built by the scoring kernel
  for (int b = tid; b < HIST1; b += SEL_THREADS) hist[b] = ghist[g * HIST1 + b];
  if (tid == 0) s_ncand = 0;
  __syncthreads();
  find_bin(hist, HIST1, k, tmp, &s_bin, &s_above);
  unsigned int prefix = (unsigned int)s_bin;
  unsigned int rank = k - s_above;  // rank of the cut key inside the bin, from the top
  int shift = 32 - HIST1_BITS;
  const unsigned int bin_count = hist[prefix];
  const bool in_lds = bin_count <= (unsigned int)CAND_CAP;

  // every wave owns a contiguous segment of candidate rows
  constexpr int NWV = SEL_THREADS / 64;
  const int n = hi - lo;
  const int seg = ((n + NWV - 1) / NWV + 63) / 64 * 64;
  const int s0 = min(lo + wave * seg, hi);
  const int s1 = min(s0 + seg, hi);

  // gather the cut bin's keys into LDS (order irrelevant: only counted); one
  // LDS atomic per wave step (ballot + in-wave rank)
  if (in_lds) {
    wave_pass_keys(sc, s0, s1, [&](int, bool valid, unsigned int key) {
      const bool take = valid && (key >> shift) == prefix;
      const unsigned long long m = __ballot(take);
      if (m) {
        const int leader = __ffsll((long long)m) - 1;
        unsigned int base = 0;
        if (lane == leader) base = atomicAdd(&s_ncand, (unsigned int)__popcll(m));
        base = __shfl(base, leader);
        if (take) cand[base + popc64(m & lanemask_lt())] = key;
      }
    });
    __syncthreads();
  }

  // digits 2 and 3 (10 bits each) over the keys matching the prefix
  for (int pass = 0; pass < 2; ++pass) {
    const int nbits = 10;
    const int nb = 1 << nbits;
    __syncthreads();
    for (int b = tid; b < nb; b += SEL_THREADS) hist[b] = 0u;
    __syncthreads();
    const int new_shift = shift - nbits;
    if (in_lds) {
      const unsigned int n = s_ncand;
      for (unsigned int i = tid; i < n; i += SEL_THREADS) {
        const unsigned int key = cand[i];
        if ((key >> shift) == prefix) atomicAdd(&hist[(key >> new_shift) & (nb - 1)], 1u);
      }
    } else {
      for (int j = lo + tid; j < hi; j += SEL_THREADS) {
        const unsigned int key = f2key(sc[j]);
        if ((key >> shift) == prefix) atomicAdd(&hist[(key >> new_shift) & (nb - 1)], 1u);
      }
    }
    __syncthreads();
    find_bin(hist, nb, rank, tmp, &s_bin, &s_above);
    prefix = (prefix << nbits) | (unsigned int)s_bin;
    rank -= s_above;
    shift = new_shift;
  }
  const unsigned int cut = prefix;        // exact key of the B'-th candidate
  const unsigned int need_ties = rank;    // ties at the cut to take, earliest rows first

  // ordered emission: each wave owns a contiguous segment of candidate rows;
  // pass 1 counts, one scan over the waves gives each segment's offsets, pass 2
  // writes in row order using ballots for the in-wave ranks.
  unsigned int cgt = 0, ctie = 0;
  wave_pass_keys(sc, s0, s1, [&](int, bool valid, unsigned int key) {
    cgt += valid && key > cut;
    ctie += valid && key == cut;
  });
  for (int m = 32; m >= 1; m >>= 1) {
    cgt += __shfl_xor(cgt, m);
    ctie += __shfl_xor(ctie, m);
  }
  if (lane == 0) {
    wave_gt[wave] = cgt;
    wave_tie[wave] = ctie;
  }
  __syncthreads();
  unsigned int gt_run = 0, tie_run = 0;
  for (int w = 0; w < wave; ++w) {
    gt_run += wave_gt[w];
    tie_run += wave_tie[w];
  }
  wave_pass_keys(sc, s0, s1, [&](int j, bool valid, unsigned int key) {
    const bool gt = valid && key > cut;
    const bool tie = valid && key == cut;
    const unsigned long long tie_mask = __ballot(tie);
    const unsigned int tie_rank = tie_run + popc64(tie_mask & lanemask_lt());
    const bool take = gt || (tie && tie_rank < need_ties);
    const unsigned long long gt_mask = __ballot(gt);
    const unsigned int gt_before = gt_run + popc64(gt_mask & lanemask_lt());
    if (take) {
      const unsigned int idx = gt_before + min(tie_rank, need_ties);
      if (idx < k) out[idx] = j;
    }
    gt_run += popc64(gt_mask);
    tie_run += popc64(tie_mask);
  });
}

template <int D>
__global__ __launch_bounds__(256) void select_gather_kernel(const SelectParams p, int rows_per_block) {
  constexpr int NCH = D / 8;
  __shared__ int src_row[256];
  const int g = blockIdx.y;
  const int n_sink_eff = min(p.n_sink, p.n_ctx);
  const int rec_lo = max(p.n_sink, p.n_ctx - p.n_recent);
  const int r0 = blockIdx.x * rows_per_block;
  const int r1 = min(r0 + rows_per_block, p.n_part);
  const int32_t* sel = p.sel_idx + (int64_t)g * p.budget;
  if (threadIdx.x < r1 - r0) {
    const int r = r0 + threadIdx.x;
    int src;
    if (r < n_sink_eff) src = r;
    else if (r < n_sink_eff + p.b_eff) src = sel[r - n_sink_eff];
    else src = rec_lo + (r - n_sink_eff - p.b_eff);
    src_row[threadIdx.x] = min(max(src, 0), p.n_ctx - 1);  // the selection only emits rows in [0, n_ctx)
  }
  __syncthreads();
  const int nchunks = (r1 - r0) * NCH * 2;
  for (int id = threadIdx.x; id < nchunks; id += 256) {
    const bool is_v = id >= (r1 - r0) * NCH;
    const int cid = is_v ? id - (r1 - r0) * NCH : id;
    const int rl = cid / NCH;
    const int ch = cid % NCH;
    const uint16_t* s = (is_v ? p.v : p.k) + (int64_t)g * p.s_head + (int64_t)src_row[rl] * p.s_pos + ch * 8;
    uint16_t* d = (is_v ? p.v_part : p.k_part) + (int64_t)g * p.sp_head + (int64_t)(r0 + rl) * p.sp_pos + ch * 8;
    *reinterpret_cast<u32x4*>(d) = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(s));
  }
}

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

size_t select_workspace_bytes(int32_t n_ctx, int32_t T, int32_t Hq, int32_t Hkv, int32_t d, int32_t budget) {
  (void)T;
  (void)Hq;
  (void)budget;
  return round256((size_t)Hkv * n_ctx * sizeof(float)) + round256((size_t)Hkv * d * sizeof(float)) +
         round256((size_t)Hkv * HIST1 * sizeof(unsigned int));
}

hipError_t launch_select(const SelectParams& p, hipStream_t stream) {
  unsigned int* hist = reinterpret_cast<unsigned int*>(p.sel_ws);
  if (p.d == 128)
    hipLaunchKernelGGL(select_prologue_kernel<128>, dim3(p.Hkv), dim3(256), 0, stream, p, hist);
  else
    hipLaunchKernelGGL(select_prologue_kernel<64>, dim3(p.Hkv), dim3(256), 0, stream, p, hist);
  if (p.n_ctx > 0) {
    // ~1024 scoring blocks over all heads, at least 256 rows each
    int chunks = (1024 + p.Hkv - 1) / p.Hkv;
    int rpb = (p.n_ctx + chunks - 1) / chunks;
    if (rpb < 256) rpb = 256;
    chunks = (p.n_ctx + rpb - 1) / rpb;
    if (p.d == 128)
      hipLaunchKernelGGL(select_score_kernel<128>, dim3(chunks, p.Hkv), dim3(256), 0, stream, p, hist, rpb);
    else
      hipLaunchKernelGGL(select_score_kernel<64>, dim3(chunks, p.Hkv), dim3(256), 0, stream, p, hist, rpb);
  }
  hipLaunchKernelGGL(select_topb_kernel, dim3(p.Hkv), dim3(SEL_THREADS), 0, stream, p, hist);
  if (p.n_part > 0) {
    const int rpb = 32;
    const int chunks = (p.n_part + rpb - 1) / rpb;
    if (p.d == 128)
      hipLaunchKernelGGL(select_gather_kernel<128>, dim3(chunks, p.Hkv), dim3(256), 0, stream, p, rpb);
    else
      hipLaunchKernelGGL(select_gather_kernel<64>, dim3(chunks, p.Hkv), dim3(256), 0, stream, p, rpb);
  }
  return hipGetLastError();
}

}  // namespace ts
