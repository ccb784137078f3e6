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
//   1. score     grid (chunks, Hkv): qbar_g in fp32 from the group's query
//                rows (copied to LDS while the first K tile is in flight),
//                then one HBM pass over K. 16 lanes x 16 B per row (d=128),
//                lane-local FMAs then a 16-lane reduction; the block also
//                histograms the top 12 bits of each candidate's
//                order-preserving key and adds its non-empty bins to the
//                head's global histogram; the blocks also clear the head's
//                second-digit histogram for pass 2.
//   2. cutbin    grid (nb, Hkv): every block finds the top-12-bit bin holding
//                the B'-th key, lists its chunk's keys in that bin, counts its
//                keys in higher bins and adds the next 10 bits of its listed
//                keys to the head's second-digit histogram; the blocks also
//                share out the -1 padding of sel_idx and the copies of the
//                sink and recent rows.
//   3. emit      grid (nb, Hkv): every block takes the second digit from that
//                histogram and the last one from the lists (exact cut), counts
//                the rows taken by earlier blocks, writes its selected rows in
//                ascending order and copies their K and V rows into the
//                partial cache; the blocks also clear the head's first-digit
//                histogram for the next call (pass 2 does it when nothing is
//                selected).
// Passes 2 and 3 read the L2-resident scores, not K.
//
// The first-digit histogram is left at zero by every call, so no clearing
// launch is needed. A workspace that does not hold a zero histogram (its
// first use, or a call that did not complete) is caught by pass 2: the
// histogram's total must be the head's candidate count, and when it is not,
// each block rebuilds the head's histogram from the scores.
//
// With the scores given (computed by the verification pass over the same
// queries), pass 2 becomes one read of the scores that fills the first-digit
// histogram.
#include "ts_device.h"
#include "ts_internal.h"

#include <cmath>

namespace ts {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int HIST1_BITS = 12;
constexpr int HIST1 = 1 << HIST1_BITS;  // bins of the first radix digit
constexpr int HIST2_BITS = 10;
constexpr int HIST2 = 1 << HIST2_BITS;  // bins of the second and third digits

__device__ inline float bf16_lo(unsigned int w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(unsigned int w) { return __uint_as_float(w & 0xffff0000u); }

__device__ inline unsigned int popc64(unsigned long long x) { return (unsigned int)__popcll(x); }

// Scoring ring: two stages of 256-row tiles, 16 waves (measured at 8B / 100K:
// 35.4 us; four stages of 128 rows: 36.0 us with 8 or 16 waves; two stages
// of 256 rows with 8 waves: 38.6 us).
constexpr int SC_ROWS = 256;    // K rows per tile
constexpr int SC_STAGES = 2;    // ring depth: one tile in flight while one is scored
constexpr int SC_WAVES = 16;    // four waves per SIMD hide the LDS and reduction latencies

// Sum over the 16 lanes of a DPP row (every lane gets the sum): rotations by
// 8, 4, 2, 1 within the row, VALU only.
__device__ inline float row16_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false));  // row_ror:8
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xf, 0xf, false));  // row_ror:4
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xf, 0xf, false));  // row_ror:2
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xf, 0xf, false));  // row_ror:1
  return x;
}

// One workgroup per chunk of rows_per_block rows of one KV head: K streams
// through an LDS ring of SC_STAGES tiles of SC_ROWS rows (asynchronous
// copies), each row is scored from LDS by LPR lanes holding 8
// channels (lane-local FMAs, then an LPR-lane reduction), and candidate rows
// are histogrammed by the top 12 bits of their order-preserving key. Before
// the first tile, the workgroup forms qbar_g itself: the group's query rows
// are copied into the ring's last slot (free until the loop refills it)
// ahead of the first K tile, so the sum runs while that tile is in flight.
template <int D>
__global__ __launch_bounds__(SC_WAVES * 64) void select_score_kernel(const SelectParams p, unsigned int* ghist,
                                                                    unsigned int* ghist2, int rows_per_block) {
  constexpr int NT = SC_WAVES * 64;
  constexpr int LPR = D / 8;                 // lanes per row
  constexpr int RPW = 64 / LPR;              // rows per wave per step
  constexpr int ROWB = D * 2;                // bytes per staged row
  constexpr int TILE_BYTES = SC_ROWS * ROWB;
  constexpr int ROWS_PER_DMA = 1024 / ROWB;
  constexpr int DPW = TILE_BYTES / 1024 / SC_WAVES;   // copies per wave per tile
  constexpr int STEPS = SC_ROWS / SC_WAVES / RPW;     // steps per wave per tile
  static_assert(DPW >= 1 && STEPS >= 1, "tile covers every wave");
  __shared__ __attribute__((aligned(1024))) unsigned char ring[SC_STAGES * TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) float qlds[256];   // q-bar of the head (one 64-lane copy)
  __shared__ unsigned int lhist[HIST1];
  const int g = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int sub = lane % LPR;
  const int rsub = lane / LPR;

  const int r0 = blockIdx.x * rows_per_block;
  const int r1 = min(r0 + rows_per_block, p.n_ctx);
  const int ntiles = r1 > r0 ? (r1 - r0 + SC_ROWS - 1) / SC_ROWS : 0;
  const int64_t row_bytes = p.s_pos * 2;
  const unsigned char* kbase = reinterpret_cast<const unsigned char*>(p.k + (int64_t)g * p.s_head);
  const unsigned int ring_off = lds_offset(ring);
  // copy j of a tile (wave w issues j = w, w + SC_WAVES, ...) covers ROWS_PER_DMA dense rows
  const unsigned int loff = (unsigned int)((wave * ROWS_PER_DMA + lane / LPR) * row_bytes) + (lane % LPR) * 16;
  const unsigned int jj_step = (unsigned int)(SC_WAVES * ROWS_PER_DMA * row_bytes);
  auto issue = [&](int t) {
    const int64_t rem = (int64_t)(r1 - r0 - t * SC_ROWS) * row_bytes;
    const unsigned int nrec = rem > 0xffffffffll ? 0xffffffffu : (unsigned int)rem;
    const i32x4 desc = buffer_desc(kbase + (int64_t)(r0 + t * SC_ROWS) * row_bytes, nrec);
    const unsigned int slot = ring_off + (unsigned int)((t % SC_STAGES) * TILE_BYTES);
#pragma unroll
    for (int jj = 0; jj < DPW; ++jj) dma16_nt(desc, loff, jj * jj_step, slot + (wave + jj * SC_WAVES) * 1024);
  };
  // qbar_g: the group's query rows, QCH at a time, go to the ring's last slot
  // by the same copy (a plain load would make the compiler wait for every
  // copy in flight); the first round's copies go out before the first K tile
  // so that a wait for them leaves that tile in flight.
  static_assert(SC_STAGES == 2, "the first round's wait counts one K tile behind the query rows");
  constexpr int QCH = TILE_BYTES / ROWB;   // query rows per round
  constexpr int QRS = NT / LPR;            // row slots (LPR threads per row)
  const int qrows = (p.Hq / p.Hkv) * p.T;
  const unsigned char* qbase = reinterpret_cast<const unsigned char*>(p.q + (int64_t)g * qrows * D);
  const unsigned int qslot = ring_off + (unsigned int)((SC_STAGES - 1) * TILE_BYTES);
  auto issue_q = [&](int c) {   // rows [c QCH, c QCH + nr) to the slot, densely
    const unsigned int bytes = (unsigned int)(min(QCH, qrows - c * QCH) * ROWB);
    const i32x4 desc = buffer_desc(qbase + (int64_t)c * QCH * ROWB, bytes);
    for (int j = wave; j < (int)((bytes + 1023) / 1024); j += SC_WAVES)
      dma16(desc, (unsigned int)(lane * 16), (unsigned int)(j * 1024), qslot + (unsigned int)(j * 1024));
  };
  issue_q(0);
  if (ntiles > 0) issue(0);
  // the head's second-digit histogram, for pass 2 (nothing reads it before)
  for (int b = blockIdx.x * NT + tid; b < HIST2; b += gridDim.x * NT) ghist2[g * HIST2 + b] = 0u;
  float qa[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};   // channels [8 sub', 8 sub' + 8) of this thread's row slots
  const int nqc = (qrows + QCH - 1) / QCH;
  for (int c = 0; c < nqc; ++c) {
    if (c > 0) {
      __syncthreads();   // the previous round's rows are read
      issue_q(c);
    }
    if (c == 0 && ntiles > 0) wait_vm<DPW>();   // copies retire in order: the rows, not the K tile
    else wait_vm<0>();
    __syncthreads();
    const int nr = min(QCH, qrows - c * QCH);
    for (int r = tid / LPR; r < nr; r += QRS) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(ring + (SC_STAGES - 1) * TILE_BYTES + r * ROWB + (tid % LPR) * 16);
      qa[0] += bf16_lo(w.x); qa[1] += bf16_hi(w.x);
      qa[2] += bf16_lo(w.y); qa[3] += bf16_hi(w.y);
      qa[4] += bf16_lo(w.z); qa[5] += bf16_hi(w.z);
      qa[6] += bf16_lo(w.w); qa[7] += bf16_hi(w.w);
    }
  }
  // row slots of a wave, then the waves, in a fixed order (deterministic);
  // the histogram's LDS holds the per-wave sums until it is cleared
  static_assert(LPR == 8 || LPR == 16, "row slots of 8 or 16 lanes");
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if constexpr (LPR == 8) qa[e] = xor_add<8>(qa[e]);
    qa[e] = xor_add<16>(qa[e]);
    qa[e] = xor_add<32>(qa[e]);
  }
  static_assert(SC_WAVES * D <= HIST1, "per-wave sums fit the histogram's LDS");
  float* qpart = reinterpret_cast<float*>(lhist);
  if (lane < LPR)
#pragma unroll
    for (int e = 0; e < 8; ++e) qpart[wave * D + lane * 8 + e] = qa[e];
  __syncthreads();
  if (tid < D) {
    float t = 0.f;
    for (int w = 0; w < SC_WAVES; ++w) t += qpart[w * D + tid];
    qlds[tid] = t;
  }
  __syncthreads();
  for (int b = tid; b < HIST1; b += NT) lhist[b] = 0u;   // ordered before the atomics by the first tile's barrier

  float* sc = p.scores + (int64_t)g * p.n_ctx;
  for (int t = 0; t < ntiles; ++t) {
    const int later = min(SC_STAGES - 2, ntiles - 1 - t);   // tiles issued after this one
    if (later >= 2) wait_vm<2 * DPW>();
    else if (later == 1) wait_vm<DPW>();
    else wait_vm<0>();
    __syncthreads();   // tile t landed for every wave; tile t-1's slot is free
    if (t + SC_STAGES - 1 < ntiles) issue(t + SC_STAGES - 1);
    const unsigned char* tl = ring + (t % SC_STAGES) * TILE_BYTES;
    float qb[8];
    {
      const f32x4 a = *reinterpret_cast<const f32x4*>(qlds + sub * 8);
      const f32x4 b = *reinterpret_cast<const f32x4*>(qlds + sub * 8 + 4);
      qb[0] = a.x; qb[1] = a.y; qb[2] = a.z; qb[3] = a.w;
      qb[4] = b.x; qb[5] = b.y; qb[6] = b.z; qb[7] = b.w;
    }
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
      const int row = (wave * STEPS + st) * RPW + rsub;   // row within the tile
      const int j = r0 + t * SC_ROWS + row;
      const u32x4 w = *reinterpret_cast<const u32x4*>(tl + row * ROWB + sub * 16);
      float acc = 0.f;
      acc = fmaf(qb[0], bf16_lo(w.x), acc);
      acc = fmaf(qb[1], bf16_hi(w.x), acc);
      acc = fmaf(qb[2], bf16_lo(w.y), acc);
      acc = fmaf(qb[3], bf16_hi(w.y), acc);
      acc = fmaf(qb[4], bf16_lo(w.z), acc);
      acc = fmaf(qb[5], bf16_hi(w.z), acc);
      acc = fmaf(qb[6], bf16_lo(w.w), acc);
      acc = fmaf(qb[7], bf16_hi(w.w), acc);
      if constexpr (LPR == 16) {
        acc = row16_sum(acc);
      } else {
#pragma unroll
        for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
      }
      if (sub == 0 && j < r1) {
        sc[j] = acc;
        if (j >= p.cand_lo && j < p.cand_hi) atomicAdd(&lhist[f2key(acc) >> (32 - HIST1_BITS)], 1u);
      }
    }
  }
  __syncthreads();
  for (int b = tid; b < HIST1; b += NT) {
    const unsigned int c = lhist[b];
    if (c) atomicAdd(&ghist[g * HIST1 + b], c);
  }
}

// First-digit histogram of the given scores of the candidate rows: one block
// per chunk of rows_per_block candidates of one KV head, LDS histogram, then
// the non-empty bins added to the head's global histogram.
__global__ __launch_bounds__(256) void select_hist_kernel(const SelectParams p, unsigned int* ghist,
                                                         unsigned int* ghist2, int rows_per_block) {
  __shared__ unsigned int lhist[HIST1];
  const int g = blockIdx.y;
  const int tid = threadIdx.x;
  for (int b = blockIdx.x * 256 + tid; b < HIST2; b += gridDim.x * 256) ghist2[g * HIST2 + b] = 0u;
  for (int b = tid; b < HIST1; b += 256) lhist[b] = 0u;
  __syncthreads();
  const int r0 = p.cand_lo + blockIdx.x * rows_per_block;
  const int r1 = min(r0 + rows_per_block, p.cand_hi);
  const float* sc = p.scores + (int64_t)g * p.n_ctx;
  constexpr int U = 8;   // loads in flight per thread
  for (int j0 = r0 + tid; j0 < r1; j0 += 256 * U) {
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = j0 + u * 256 < r1 ? sc[j0 + u * 256] : 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (j0 + u * 256 < r1) atomicAdd(&lhist[f2key(v[u]) >> (32 - HIST1_BITS)], 1u);
  }
  __syncthreads();
  for (int b = tid; b < HIST1; b += 256) {
    const unsigned int c = lhist[b];
    if (c) atomicAdd(&ghist[g * HIST1 + b], c);
  }
}

// Workspace after the scores (all 256-byte aligned):
//   hist   [Hkv][HIST1]     first-digit histogram (filled by the scoring pass)
//   hist2  [Hkv][HIST2]     second-digit histogram of the cut bin's keys
//   cut1   [Hkv][2]         the cut bin of the first digit and the keys above it
//   ccnt   [Hkv][NB_MAX][2] per block: cut-bin keys collected, keys in higher bins
//   cand   [Hkv][n_ctx]     the cut-bin keys, block b's at its chunk's rows
constexpr int NB_MAX = 64;   // blocks per head in the parallel passes
constexpr int PT = 256;      // threads per block of the parallel passes

__host__ __device__ inline size_t round256(size_t x) { return (x + 255) / 256 * 256; }

struct SelWs {
  unsigned int* hist;
  unsigned int* hist2;
  unsigned int* cut1;
  unsigned int* ccnt;
  unsigned int* cand;
};

__host__ __device__ inline SelWs carve(int32_t* base, int Hkv, int n_ctx) {
  char* w = reinterpret_cast<char*>(base);
  SelWs s;
  s.hist = reinterpret_cast<unsigned int*>(w);
  w += round256((size_t)Hkv * HIST1 * 4);
  s.hist2 = reinterpret_cast<unsigned int*>(w);
  w += round256((size_t)Hkv * HIST2 * 4);
  s.cut1 = reinterpret_cast<unsigned int*>(w);
  w += round256((size_t)Hkv * 2 * 4);
  s.ccnt = reinterpret_cast<unsigned int*>(w);
  w += round256((size_t)Hkv * NB_MAX * 2 * 4);
  s.cand = reinterpret_cast<unsigned int*>(w);
  (void)n_ctx;
  return s;
}

size_t sel_ws_bytes(int Hkv, int n_ctx) {
  return round256((size_t)Hkv * HIST1 * 4) + round256((size_t)Hkv * HIST2 * 4) + round256((size_t)Hkv * 2 * 4) +
         round256((size_t)Hkv * NB_MAX * 2 * 4) + round256((size_t)Hkv * (n_ctx > 0 ? n_ctx : 1) * 4);
}

// Block-wide exclusive scan over NT threads; returns the prefix and the total.
// `tmp` holds one slot per wave.
template <int NT>
__device__ inline unsigned int block_exclusive_scan(unsigned int x, unsigned int* tmp, unsigned int* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const unsigned int incl = wave_incl_scan(x);
  if (lane == 63) tmp[wave] = incl;
  __syncthreads();
  unsigned int wave_prefix = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
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
// higher bins). Each thread owns nbins / NT consecutive bins.
template <int NT>
__device__ inline void find_bin(const unsigned int* hist, int nbins, unsigned int k, unsigned int* tmp, int* bin_out,
                                unsigned int* above_out, unsigned int* total_out = nullptr) {
  const int per = nbins / NT;
  const int hi_bin = nbins - 1 - threadIdx.x * per;   // thread t covers the t-th group from the top
  unsigned int s = 0;
  for (int i = 0; i < per; ++i) s += hist[hi_bin - i];
  unsigned int total;
  const unsigned int before = block_exclusive_scan<NT>(s, tmp, &total);
  if (total_out) *total_out = total;
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

// Candidate rows [lo, hi) are cut into NB chunks of `chunk` rows (a multiple
// of 64); block b of a head owns chunk b.
__device__ inline void chunk_of(const SelectParams& p, int nb, int b, int* c0, int* c1) {
  const int n = p.cand_hi - p.cand_lo;
  const int chunk = ((n + nb - 1) / nb + 63) / 64 * 64;
  *c0 = min(p.cand_lo + b * chunk, p.cand_hi);
  *c1 = min(*c0 + chunk, p.cand_hi);
}

constexpr int RPT = 16;        // consecutive rows per thread in one sub-chunk of a parallel pass
constexpr int SUB = PT * RPT;  // rows per sub-chunk

// hist (HIST1 u32 in LDS) <- src, with every thread's 16-byte loads issued together.
template <int NT>
__device__ inline void load_hist(unsigned int* hist, const unsigned int* src) {
  constexpr int PER = HIST1 / 4 / NT;
  u32x4 v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) v[i] = reinterpret_cast<const u32x4*>(src)[threadIdx.x + i * NT];
#pragma unroll
  for (int i = 0; i < PER; ++i) reinterpret_cast<u32x4*>(hist)[threadIdx.x + i * NT] = v[i];
}

// Keys of rows j0 .. j0+RPT-1. Rows at or past c1 are invalid (every caller
// tests j < c1) and read row c1 - 1 (c1 >= 1), so the loads issue without
// branches.
__device__ inline void load_keys(const float* sc, int j0, int c1, unsigned int (&key)[RPT]) {
  float v[RPT];
#pragma unroll
  for (int e = 0; e < RPT; ++e) v[e] = sc[min(j0 + e, c1 - 1)];
#pragma unroll
  for (int e = 0; e < RPT; ++e) key[e] = f2key(v[e]);
}

constexpr int CAND_CAP = 8192;   // cut-bin keys refined in LDS (more are refined from L2)

// Copy rows of K and V of head g into the partial cache: item i of `n` is
// 16-byte chunk i % RCH of pair i / RCH, pairs (src, dst) given by `pair`.
// Items item0, item0 + stride, ... are this thread's; CP of them are in
// flight together (loads first, then stores).
template <int D, typename F>
__device__ inline void copy_rows(const SelectParams& p, int g, int n, int item0, int stride, F&& pair) {
  constexpr int NCH = D / 8, RCH = 2 * NCH, CP = 16;
  for (int base = item0; base < n * RCH; base += stride * CP) {
    u32x4 val[CP];
    uint16_t* dst[CP];
#pragma unroll
    for (int u = 0; u < CP; ++u) {
      const int id = base + u * stride;
      dst[u] = nullptr;
      if (id < n * RCH) {
        int src_row, dst_row;
        pair(id / RCH, &src_row, &dst_row);
        const int c = id % RCH;
        const bool is_v = c >= NCH;
        const int ch = is_v ? c - NCH : c;
        const uint16_t* src = (is_v ? p.v : p.k) + (int64_t)g * p.s_head + (int64_t)src_row * p.s_pos + ch * 8;
        dst[u] = (is_v ? p.v_part : p.k_part) + (int64_t)g * p.sp_head + (int64_t)dst_row * p.sp_pos + ch * 8;
        val[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));
      }
    }
    // one wait for all the loads: stores count in the same counter, so the
    // compiler's wait before each store would otherwise hold it for the
    // previous store's acknowledgement
#pragma unroll
    for (int u = 0; u < CP; ++u) asm volatile("" ::"v"(val[u]));
#pragma unroll
    for (int u = 0; u < CP; ++u)
      if (dst[u]) *reinterpret_cast<u32x4*>(dst[u]) = val[u];
  }
}

// Pass 1 of the selection. Every block of a head: the first-digit bin holding
// the B'-th key (from the scoring histogram; every block finds the same one),
// the list of its chunk's keys in that bin in cand[g] at the chunk's own rows
// (unordered; slots from an LDS counter, so no global atomic is contended),
// its count of keys in higher bins, and the next 10 bits of its listed keys
// added to the head's second-digit histogram. The blocks of a head also share
// out the -1 padding of sel_idx and the copies of the sink and recent rows,
// which do not depend on the cut.
template <int D>
__global__ __launch_bounds__(PT) void select_cutbin_kernel(const SelectParams p, int nb) {
  __shared__ __attribute__((aligned(16))) unsigned int hist[HIST1];
  __shared__ unsigned int h2[HIST2];
  __shared__ unsigned int tmp[PT / 64];
  __shared__ int s_bin;
  __shared__ unsigned int s_above, s_n, s_hi;
  const int g = blockIdx.y;
  const unsigned int k = (unsigned int)p.b_eff;
  const SelWs ws = carve(p.sel_ws, p.Hkv, p.n_ctx);
  const int tid = threadIdx.x, lane = tid & 63;
  int c0, c1;
  chunk_of(p, nb, blockIdx.x, &c0, &c1);
  const float* sc = p.scores + (int64_t)g * p.n_ctx;
  unsigned int* cand = ws.cand + (int64_t)g * p.n_ctx + c0;
  // the first sub-chunk's keys are loaded together with the histogram
  unsigned int key[RPT];
  if (k > 0) {
    load_keys(sc, c0 + RPT * tid, c1, key);
    load_hist<PT>(hist, ws.hist + g * HIST1);
  }
  for (int b = tid; b < HIST2; b += PT) h2[b] = 0u;
  if (tid == 0) s_n = s_hi = 0;
  // padding and sink / recent copies, strided over the head's blocks: every
  // thread's first 16-byte item is loaded now and stored at the end, so its
  // latency hides behind the pass; further items (long sink / recent ranges)
  // are copied at the end
  int32_t* out = p.sel_idx + (int64_t)g * p.budget;
  for (int i = (int)k + blockIdx.x * PT + tid; i < p.budget; i += nb * PT) out[i] = -1;
  const int n_sink_eff = min(p.n_sink, p.n_ctx);
  const int rec_lo = max(p.n_sink, p.n_ctx - p.n_recent);
  const int n_copy = n_sink_eff + (p.n_ctx - rec_lo > 0 ? p.n_ctx - rec_lo : 0);
  auto pair = [&](int r, int* src, int* dst) {
    *src = r < n_sink_eff ? r : rec_lo + (r - n_sink_eff);
    *dst = r < n_sink_eff ? r : n_sink_eff + (int)k + (r - n_sink_eff);
  };
  const int item0 = blockIdx.x * PT + tid, stride = nb * PT;
  u32x4 first_v = {0u, 0u, 0u, 0u};
  uint16_t* first_dst = nullptr;
  {
    constexpr int NCH = D / 8, RCH = 2 * NCH;
    if (item0 < n_copy * RCH) {
      int src_row, dst_row;
      pair(item0 / RCH, &src_row, &dst_row);
      const int c = item0 % RCH;
      const bool is_v = c >= NCH;
      const int ch = is_v ? c - NCH : c;
      first_v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
          (is_v ? p.v : p.k) + (int64_t)g * p.s_head + (int64_t)src_row * p.s_pos + ch * 8));
      first_dst = (is_v ? p.v_part : p.k_part) + (int64_t)g * p.sp_head + (int64_t)dst_row * p.sp_pos + ch * 8;
    }
  }
  auto finish_copies = [&]() {
    if (first_dst) *reinterpret_cast<u32x4*>(first_dst) = first_v;
    copy_rows<D>(p, g, n_copy, item0 + stride, stride, pair);
  };
  if (k == 0) {
    // nothing is selected, so no later pass runs: clear the first-digit
    // histogram here (no block of this pass reads it)
    for (int b = blockIdx.x * PT + tid; b < HIST1; b += nb * PT) ws.hist[g * HIST1 + b] = 0u;
    finish_copies();
    return;
  }
  bar();
  unsigned int total = 0;
  find_bin<PT>(hist, HIST1, k, tmp, &s_bin, &s_above, &total);
  if (total != (unsigned int)(p.cand_hi - p.cand_lo)) {
    // the histogram did not start at zero: count this head's candidates here
    for (int b = tid; b < HIST1; b += PT) hist[b] = 0u;
    bar();
    for (int j = p.cand_lo + tid; j < p.cand_hi; j += PT) atomicAdd(&hist[f2key(sc[j]) >> (32 - HIST1_BITS)], 1u);
    bar();
    find_bin<PT>(hist, HIST1, k, tmp, &s_bin, &s_above);
  }
  const unsigned int bin = (unsigned int)s_bin;
  constexpr int SH2 = 32 - HIST1_BITS - HIST2_BITS;
  unsigned int n_hi = 0;   // this thread's keys in higher first-digit bins
  for (int s0 = c0; s0 < c1; s0 += SUB) {
    const int j0 = s0 + RPT * tid;
    if (s0 != c0) load_keys(sc, j0, c1, key);
    unsigned int nc = 0;
#pragma unroll
    for (int e = 0; e < RPT; ++e) {
      const unsigned int kb = key[e] >> (32 - HIST1_BITS);
      nc += j0 + e < c1 && kb == bin;
      n_hi += j0 + e < c1 && kb > bin;
    }
    // in-wave exclusive prefix of the list lengths; one LDS atomic per wave
    const unsigned int incl = wave_incl_scan(nc);
    unsigned int base = 0;
    if (lane == 63 && incl) base = atomicAdd(&s_n, incl);
    base = lane_value(base, 63) + incl - nc;
    if (nc) {
#pragma unroll
      for (int e = 0; e < RPT; ++e)
        if (j0 + e < c1 && (key[e] >> (32 - HIST1_BITS)) == bin) {
          cand[base++] = key[e];
          atomicAdd(&h2[(key[e] >> SH2) & (HIST2 - 1)], 1u);
        }
    }
  }
  n_hi = wave_reduce(n_hi, OpAdd());
  if (lane == 0) atomicAdd(&s_hi, n_hi);
  bar();
  for (int b = tid; b < HIST2; b += PT) {
    const unsigned int c = h2[b];
    if (c) atomicAdd(&ws.hist2[g * HIST2 + b], c);
  }
  if (tid == 0) {
    ws.ccnt[(g * NB_MAX + blockIdx.x) * 2 + 0] = s_n;
    ws.ccnt[(g * NB_MAX + blockIdx.x) * 2 + 1] = s_hi;
    if (blockIdx.x == 0) {
      ws.cut1[g * 2 + 0] = bin;
      ws.cut1[g * 2 + 1] = s_above;
    }
  }
  finish_copies();
}

// Pass 2: exact cut, ordered emission and gather; grid (nb, Hkv).
// Every block of a head derives the same cut: the first-digit bin and the
// count above it from pass 1, the second digit from the head's second-digit
// histogram, and the last 10 bits from the lists of the first-digit bin's
// keys (blocks' lists back to back, in LDS when they fit) give the exact cut
// key and how many keys equal to it are taken (the earliest rows). The rows
// above the cut and at the cut in earlier blocks follow from those blocks'
// higher-bin counts and lists. Inside its chunk, sub-chunks of SUB rows are
// ranked by one block scan (rows above and at the cut, packed 16 + 16 bits),
// so selected rows come out ascending with consecutive output slots; the
// block copies their K and V rows into the partial cache.
template <int D>
__global__ __launch_bounds__(PT) void select_emit_kernel(const SelectParams p, int nb) {
  __shared__ __attribute__((aligned(16))) unsigned int hist[HIST2];
  __shared__ unsigned int cand_l[CAND_CAP];
  __shared__ int srcs[SUB];
  __shared__ unsigned int tmp[PT / 64];
  __shared__ unsigned int seg_off[NB_MAX + 1], seg_c0[NB_MAX], seg_hi[NB_MAX];
  __shared__ int s_bin;
  __shared__ unsigned int s_above, s_gt, s_tie, s_bin1, s_above1;
  const int g = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int k = p.b_eff;
  const int n_sink_eff = min(p.n_sink, p.n_ctx);
  int32_t* out = p.sel_idx + (int64_t)g * p.budget;
  const SelWs ws = carve(p.sel_ws, p.Hkv, p.n_ctx);
  int c0, c1;
  chunk_of(p, nb, blockIdx.x, &c0, &c1);
  const float* sc = p.scores + (int64_t)g * p.n_ctx;
  // pass 2 has read the first-digit histogram: leave it at zero for the next call
  for (int b = blockIdx.x * PT + tid; b < HIST1; b += nb * PT) ws.hist[g * HIST1 + b] = 0u;
  // Every load the cut needs goes out at once: lane b of every wave takes
  // block b's list length and higher-bin count, then the second-digit
  // histogram, each wave the first 64 slots of the lists of blocks wave,
  // wave + 4, ... (read before their lengths are known; slots past a list's
  // end are dropped) and this block's keys.
  const unsigned int* cand_g = ws.cand + (int64_t)g * p.n_ctx;
  unsigned int cl = 0, hl = 0;   // lane b < nb: block b's list length, its keys in higher first-digit bins
  if (lane < nb) {
    const uint2 v = *reinterpret_cast<const uint2*>(ws.ccnt + (g * NB_MAX + lane) * 2);
    cl = v.x;
    hl = v.y;
  }
  constexpr int PER = HIST2 / 4 / PT;
  u32x4 h2v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) h2v[i] = reinterpret_cast<const u32x4*>(ws.hist2 + g * HIST2)[tid + i * PT];
  int lc0, lc1;   // lane b < nb: block b's chunk
  chunk_of(p, nb, lane < nb ? lane : 0, &lc0, &lc1);
  constexpr int SPEC = NB_MAX / (PT / 64);   // lists per wave
  unsigned int spec[SPEC];
#pragma unroll
  for (int u = 0; u < SPEC; ++u) {
    const int b = wave + u * (PT / 64);
    if (b < nb) {
      const int bc0 = __builtin_amdgcn_readlane(lc0, b);
      spec[u] = cand_g[min(bc0 + lane, p.n_ctx - 1)];
    }
  }
  unsigned int key[RPT];
  load_keys(sc, c0 + RPT * tid, c1, key);
#pragma unroll
  for (int i = 0; i < PER; ++i) reinterpret_cast<u32x4*>(hist)[tid + i * PT] = h2v[i];
  // list offsets: every wave scans the list lengths (lanes >= nb hold 0)
  const unsigned int incl = wave_incl_scan(cl);
  const unsigned int loff = incl - cl;   // lane b: offset of block b's list in the concatenation
  const unsigned int n = __builtin_amdgcn_readlane(incl, 63);
  if (wave == 0) {
    if (lane < nb) {
      seg_off[lane] = loff;
      seg_c0[lane] = (unsigned int)lc0;
      seg_hi[lane] = hl;
    }
    if (lane == 63) seg_off[nb] = n;
    if (lane == 0) {
      s_gt = s_tie = 0;
      s_bin1 = ws.cut1[g * 2 + 0];
      s_above1 = ws.cut1[g * 2 + 1];
    }
  }
  auto seg_of = [&](unsigned int i) {   // list owning key i: the last b with seg_off[b] <= i
    int lo = 0, hi = nb - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (seg_off[mid] <= i) lo = mid; else hi = mid - 1;
    }
    return lo;
  };
  auto key_at = [&](unsigned int i) {
    const int b = seg_of(i);
    return cand_g[seg_c0[b] + (i - seg_off[b])];
  };
  const bool in_lds = n <= (unsigned int)CAND_CAP;
  if (in_lds) {
    // the speculative slots that lie inside their list, then the lists' slots
    // past 64 in 64-slot pieces (piece q of the concatenation of those tails
    // belongs to the first block whose pieces end after q)
#pragma unroll
    for (int u = 0; u < SPEC; ++u) {
      const int b = wave + u * (PT / 64);
      if (b < nb) {
        const unsigned int len = __builtin_amdgcn_readlane(cl, b);
        if ((unsigned int)lane < len) cand_l[__builtin_amdgcn_readlane(loff, b) + lane] = spec[u];
      }
    }
    const unsigned int np = cl > 64 ? (cl - 1) / 64 : 0;   // pieces past the first 64 slots
    const unsigned int pend = wave_incl_scan(np);
    const unsigned int n_pieces = __builtin_amdgcn_readlane(pend, 63);
    constexpr int BATCH = 8;
    for (unsigned int q0 = wave; q0 < n_pieces; q0 += (PT / 64) * BATCH) {
      unsigned int v[BATCH];
      int dst[BATCH];
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        const unsigned int q = q0 + u * (PT / 64);
        dst[u] = -1;
        if (q < n_pieces) {
          const int b = (int)popc64(__ballot(pend <= q));
          const unsigned int i = 64u * (1u + q - (__builtin_amdgcn_readlane(pend, b) - __builtin_amdgcn_readlane(np, b))) +
                                 (unsigned int)lane;
          if (i < __builtin_amdgcn_readlane(cl, b)) {
            v[u] = cand_g[__builtin_amdgcn_readlane(lc0, b) + i];
            dst[u] = (int)(__builtin_amdgcn_readlane(loff, b) + i);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < BATCH; ++u)
        if (dst[u] >= 0) cand_l[dst[u]] = v[u];
    }
  }
  bar();   // histogram, list offsets and lists in LDS
  // second digit from the head's histogram of the cut bin's keys
  unsigned int rank = (unsigned int)k - s_above1;   // rank of the cut key inside the first-digit bin
  find_bin<PT>(hist, HIST2, rank, tmp, &s_bin, &s_above);
  unsigned int prefix = (s_bin1 << HIST2_BITS) | (unsigned int)s_bin;
  rank -= s_above;
  bar();   // every thread has read the histogram (and the lists are in LDS)
  // last digit from the listed keys with that prefix
  constexpr int SH = 32 - HIST1_BITS - HIST2_BITS;
  for (int b = tid; b < HIST2; b += PT) hist[b] = 0u;
  bar();
  for (unsigned int i = tid; i < n; i += PT) {
    const unsigned int kk = in_lds ? cand_l[i] : key_at(i);
    if ((kk >> SH) == prefix) atomicAdd(&hist[kk & (HIST2 - 1)], 1u);
  }
  bar();
  find_bin<PT>(hist, HIST2, rank, tmp, &s_bin, &s_above);
  const unsigned int cut = (prefix << SH) | (unsigned int)s_bin, need = rank - s_above;
  // rows above / at the cut in earlier blocks: their higher-bin counts plus
  // their listed keys above / equal to the cut
  {
    unsigned int gt = 0, tie = 0;
    const unsigned int n_before = seg_off[blockIdx.x];
    for (unsigned int i = tid; i < n_before; i += PT) {
      const unsigned int kk = in_lds ? cand_l[i] : key_at(i);
      gt += kk > cut;
      tie += kk == cut;
    }
    if (tid < (int)blockIdx.x) gt += seg_hi[tid];
    gt = wave_reduce(gt, OpAdd());
    tie = wave_reduce(tie, OpAdd());
    if (lane == 0) {
      atomicAdd(&s_gt, gt);
      atomicAdd(&s_tie, tie);
    }
  }
  bar();
  unsigned int gt_run = s_gt, tie_run = s_tie;
  for (int s0 = c0; s0 < c1; s0 += SUB) {
    const int j0 = s0 + RPT * tid;
    if (s0 != c0) load_keys(sc, j0, c1, key);
    unsigned int ngt = 0, ntie = 0;
#pragma unroll
    for (int e = 0; e < RPT; ++e) {
      const int j = j0 + e;
      ngt += j < c1 && key[e] > cut;
      ntie += j < c1 && key[e] == cut;
    }
    unsigned int tot;
    const unsigned int pre = block_exclusive_scan<PT>(ngt | (ntie << 16), tmp, &tot);
    const unsigned int base = gt_run + min(tie_run, need);   // output slot of this sub-chunk's first take
    unsigned int gt_i = gt_run + (pre & 0xffffu), tie_i = tie_run + (pre >> 16);
#pragma unroll
    for (int e = 0; e < RPT; ++e) {
      const int j = j0 + e;
      const bool gt = j < c1 && key[e] > cut;
      const bool tie = j < c1 && key[e] == cut;
      if (gt || (tie && tie_i < need)) {
        const unsigned int idx = gt_i + min(tie_i, need);
        if (idx < (unsigned int)k) srcs[idx - base] = j;
      }
      gt_i += gt;
      tie_i += tie;
    }
    gt_run += tot & 0xffffu;
    tie_run += tot >> 16;
    const unsigned int end = min(gt_run + min(tie_run, need), (unsigned int)k);
    bar();
    copy_rows<D>(p, g, (int)(end - base), tid, PT, [&](int i, int* src, int* dst) {
      *src = srcs[i];
      *dst = n_sink_eff + (int)base + i;
    });
    // the indices go out after the row copies, whose loads would otherwise
    // wait for these stores
    for (int i = tid; i < (int)(end - base); i += PT) out[base + i] = srcs[i];
    bar();
  }
}

}  // namespace

int select_blocks_per_head(int32_t n_ctx, int32_t Hkv, int32_t n_sink, int32_t n_recent) {
  const int lo = n_sink < n_ctx ? n_sink : n_ctx;
  const int hi = n_ctx - n_recent > lo ? n_ctx - n_recent : lo;
  const int n = hi - lo;
  // about two blocks per compute unit over all heads (the emit pass holds two
  // per CU): with many KV heads each block's share of the ranking and the
  // gather halves (32 heads: 183 against 193 µs per call); no change at 8 heads
  int nb = (512 + Hkv - 1) / Hkv;
  const int by_rows = (n + 1023) / 1024;    // at least 1024 rows per block
  if (nb > by_rows) nb = by_rows;
  if (nb > NB_MAX) nb = NB_MAX;
  if (nb < 1) nb = 1;
  return nb;
}

size_t select_workspace_bytes(int32_t n_ctx, int32_t T, int32_t Hq, int32_t Hkv, int32_t d, int32_t budget) {
  (void)T;
  (void)Hq;
  (void)budget;
  (void)d;
  return round256((size_t)Hkv * n_ctx * sizeof(float)) + sel_ws_bytes(Hkv, n_ctx);
}

size_t select_passes_workspace_bytes(int32_t n_ctx, int32_t Hkv) { return sel_ws_bytes(Hkv, n_ctx); }

hipError_t launch_select(const SelectParams& p, hipStream_t stream) {
  const SelWs ws = carve(p.sel_ws, p.Hkv, p.n_ctx);
  if (p.scores_given) {
    const int n_cand = p.cand_hi - p.cand_lo;
    if (n_cand > 0) {
      int chunks = (256 + p.Hkv - 1) / p.Hkv;
      int rpb = (n_cand + chunks - 1) / chunks;
      if (rpb < 2048) rpb = 2048;
      chunks = (n_cand + rpb - 1) / rpb;
      hipLaunchKernelGGL(select_hist_kernel, dim3(chunks, p.Hkv), dim3(256), 0, stream, p, ws.hist, ws.hist2, rpb);
    }
  }
  if (!p.scores_given && p.n_ctx > 0) {
    // about one scoring workgroup per compute unit over all heads, at least
    // one tile each
    int chunks = (256 + p.Hkv - 1) / p.Hkv;
    int rpb = (p.n_ctx + chunks - 1) / chunks;
    if (rpb < SC_ROWS) rpb = SC_ROWS;
    chunks = (p.n_ctx + rpb - 1) / rpb;
    if (p.d == 128)
      hipLaunchKernelGGL(select_score_kernel<128>, dim3(chunks, p.Hkv), dim3(SC_WAVES * 64), 0, stream, p, ws.hist,
                         ws.hist2, rpb);
    else
      hipLaunchKernelGGL(select_score_kernel<64>, dim3(chunks, p.Hkv), dim3(SC_WAVES * 64), 0, stream, p, ws.hist,
                         ws.hist2, rpb);
  }
  // the cut-bin pass always runs: it also pads sel_idx and copies the sink and recent rows
  const int nb = select_blocks_per_head(p.n_ctx, p.Hkv, p.n_sink, p.n_recent);
  if (p.d == 128)
    hipLaunchKernelGGL(select_cutbin_kernel<128>, dim3(nb, p.Hkv), dim3(PT), 0, stream, p, nb);
  else
    hipLaunchKernelGGL(select_cutbin_kernel<64>, dim3(nb, p.Hkv), dim3(PT), 0, stream, p, nb);
  if (p.b_eff > 0) {
    if (p.d == 128)
      hipLaunchKernelGGL(select_emit_kernel<128>, dim3(nb, p.Hkv), dim3(PT), 0, stream, p, nb);
    else
      hipLaunchKernelGGL(select_emit_kernel<64>, dim3(nb, p.Hkv), dim3(PT), 0, stream, p, nb);
  }
  return hipGetLastError();
}

}  // namespace ts
