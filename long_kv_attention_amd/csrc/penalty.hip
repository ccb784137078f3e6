// Contextual penalty, temperature, min-p and top-p over the vocabulary, for
// CDNA4 (gfx950).
//
// What is computed (TokenSwift summary §3.4, Appendix D.1, Appendix F.1;
// defaults from the reproducibility checklist's Table 11): per row, the
// windowed repetition penalty on each distinct recent id, division by the
// temperature, softmax, the top-p set (smallest prefix of the (p desc, id
// asc) order whose mass exceeds top_p, i.e. keep i iff the mass before i is at
// most top_p), the min-p set (p_i >= min_p * max p), their intersection, the
// renormalised probabilities and an inverse-CDF token for a given u.
//
// Every row is split into nb chunks of ids, one 256-thread workgroup each, so
// a few rows still spread over the whole chip. Passes (one launch each, in
// stream order; the row's z stays in L2 / the last-level cache after the
// first):
//   1. z       window ids of the chunk -> LDS bitmap (set semantics makes
//              duplicates harmless); penalty + temperature -> logits_out; the
//              chunk's max. Also clears the row's mass histogram.
//   2. hist    row max from the chunk maxima; e_i = exp(z_i - max) as 2^-40
//              fixed point; mass and count histogram over the top 12 bits of
//              the order-preserving key of z (integer atomics, so the sums do
//              not depend on timing); the chunk's total mass.
//   3. cutbin  every workgroup finds the bin where the mass from the top
//              crosses top_p * total and lists its chunk's keys in that bin.
//   4. keep    every workgroup refines the lists by two 10-bit radix digits
//              (mass histograms) to the exact cut key, the mass above it and
//              how many of its ties (ids ascending) stay; keep mask (top-p and
//              min-p) and the chunk's kept mass.
//   5. probs   renormalised probabilities; the workgroup whose kept-mass range
//              holds u * total finds the token by an ordered scan.
// Passes 2-3 and the refinement are skipped when top_p >= 1, pass 5 when
// neither probs nor a token is requested.
#include "ts_internal.h"

#include <climits>
#include <cmath>

namespace ts {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned long long u64x2 __attribute__((ext_vector_type(2)));

constexpr int PB = 256;                 // threads per workgroup
constexpr int NW = PB / 64;
constexpr int NBR_MAX = 64;             // workgroups per row
constexpr int H1_BITS = 12;
constexpr int H1 = 1 << H1_BITS;
constexpr int MAX_V = 262144;
constexpr int RPT = 16;                 // 64-id steps per wave in an ordered sub-chunk
constexpr int SEGW = 64 * RPT;          // ids per wave segment of a sub-chunk
constexpr int SUBC = PB * RPT;          // ids per ordered sub-chunk (NW segments, ascending)
constexpr int CAND_CAP = 8192;          // cut-bin keys refined in LDS (more are refined from L2)
constexpr float FIX_SCALE = 1099511627776.0f;  // 2^40

__device__ inline unsigned int f2key(float f) {
  const unsigned int u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ inline float key2f(unsigned int k) {
  const unsigned int u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}
__device__ inline unsigned long long to_fix(float e) { return (unsigned long long)(e * FIX_SCALE); }

__host__ __device__ inline size_t round256(size_t x) { return (x + 255) / 256 * 256; }

// Workspace (256-byte aligned pieces):
//   hmass [rows][H1] u64, hcnt [rows][H1] u32   the row's first-digit histogram
//   bmax  [rows][NBR_MAX] f32                  chunk maxima of z
//   zs    [rows][NBR_MAX] u64                  chunk masses (fixed point)
//   ccnt  [rows][NBR_MAX] u32                  cut-bin keys listed by each chunk
//   km    [rows][NBR_MAX] f32                  chunk kept masses
//   tie0  [rows][NBR_MAX] u32                  ties at the cut in earlier chunks
//   cut   [rows][4] u32                        cut key, ties kept, ties in all
//   cand  [rows][V] u32                        the cut-bin keys, chunk b's at its ids
struct PenWs {
  unsigned long long* hmass;
  unsigned int* hcnt;
  float* bmax;
  unsigned long long* zs;
  unsigned int* ccnt;
  float* km;
  unsigned int* tie0;
  unsigned int* cut;
  unsigned int* cand;
};

__host__ __device__ inline PenWs carve(void* base, int rows) {
  char* w = static_cast<char*>(base);
  PenWs s;
  s.hmass = reinterpret_cast<unsigned long long*>(w);
  w += round256((size_t)rows * H1 * 8);
  s.hcnt = reinterpret_cast<unsigned int*>(w);
  w += round256((size_t)rows * H1 * 4);
  s.bmax = reinterpret_cast<float*>(w);
  w += round256((size_t)rows * NBR_MAX * 4);
  s.zs = reinterpret_cast<unsigned long long*>(w);
  w += round256((size_t)rows * NBR_MAX * 8);
  s.ccnt = reinterpret_cast<unsigned int*>(w);
  w += round256((size_t)rows * NBR_MAX * 4);
  s.km = reinterpret_cast<float*>(w);
  w += round256((size_t)rows * NBR_MAX * 4);
  s.tie0 = reinterpret_cast<unsigned int*>(w);
  w += round256((size_t)rows * NBR_MAX * 4);
  s.cut = reinterpret_cast<unsigned int*>(w);
  w += round256((size_t)rows * 4 * 4);
  s.cand = reinterpret_cast<unsigned int*>(w);
  return s;
}

size_t pen_ws_bytes(int rows, int V) {
  return round256((size_t)rows * H1 * 8) + round256((size_t)rows * H1 * 4) + round256((size_t)rows * NBR_MAX * 4) +
         round256((size_t)rows * NBR_MAX * 8) + 3 * round256((size_t)rows * NBR_MAX * 4) +
         round256((size_t)rows * 4 * 4) + round256((size_t)rows * V * 4);
}

// Chunk b of nb over ids [0, V): a multiple of 64 ids.
__device__ inline void chunk_of(int V, int nb, int b, int* i0, int* i1) {
  const int chunk = ((V + nb - 1) / nb + 63) / 64 * 64;
  *i0 = min(b * chunk, V);
  *i1 = min(*i0 + chunk, V);
}

// ---- block reductions (fixed order: results do not depend on timing) ----
__device__ inline float block_max(float x, float* red) {
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < NW; ++w) r = fmaxf(r, red[w]);
  __syncthreads();
  return r;
}

template <typename T>
__device__ inline T block_sum(T x, T* red) {
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  T r = red[0];
  for (int w = 1; w < NW; ++w) r += red[w];
  __syncthreads();
  return r;
}

// Exclusive prefix over threads (thread order); *total gets the sum.
template <typename T>
__device__ inline T block_scan(T x, T* red, T* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  T incl = x;
  for (int off = 1; off < 64; off <<= 1) {
    const T y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) red[wave] = incl;
  __syncthreads();
  T pre = 0, tot = 0;
  for (int w = 0; w < NW; ++w) {
    if (w < wave) pre += red[w];
    tot += red[w];
  }
  __syncthreads();
  *total = tot;
  return pre + incl - x;
}

// Row maximum of z from the chunk maxima (one wave loads them).
__device__ inline float row_max(const PenWs& ws, int row, int nb, float* red) {
  if (threadIdx.x < 64) {
    float m = (int)threadIdx.x < nb ? ws.bmax[row * NBR_MAX + threadIdx.x] : -INFINITY;
    for (int s = 32; s >= 1; s >>= 1) m = fmaxf(m, __shfl_xor(m, s));
    if (threadIdx.x == 0) red[0] = m;
  }
  __syncthreads();
  const float r = red[0];
  __syncthreads();
  return r;
}

// Row mass (fixed point) from the chunk masses.
__device__ inline unsigned long long row_mass(const PenWs& ws, int row, int nb, unsigned long long* red) {
  if (threadIdx.x < 64) {
    unsigned long long m = (int)threadIdx.x < nb ? ws.zs[row * NBR_MAX + threadIdx.x] : 0ull;
    for (int s = 32; s >= 1; s >>= 1) m += __shfl_xor(m, s);
    if (threadIdx.x == 0) red[0] = m;
  }
  __syncthreads();
  const unsigned long long r = red[0];
  __syncthreads();
  return r;
}

// LDS copy of the row's histogram, every thread's loads issued together.
__device__ inline void load_hist(unsigned long long* hmass, unsigned int* hcnt, const PenWs& ws, int row) {
  constexpr int PM = H1 / 2 / PB, PC = H1 / 4 / PB;
  u64x2 m[PM];
  u32x4 c[PC];
  const u64x2* sm = reinterpret_cast<const u64x2*>(ws.hmass + (size_t)row * H1);
  const u32x4* scnt = reinterpret_cast<const u32x4*>(ws.hcnt + (size_t)row * H1);
#pragma unroll
  for (int i = 0; i < PM; ++i) m[i] = sm[threadIdx.x + i * PB];
#pragma unroll
  for (int i = 0; i < PC; ++i) c[i] = scnt[threadIdx.x + i * PB];
#pragma unroll
  for (int i = 0; i < PM; ++i) reinterpret_cast<u64x2*>(hmass)[threadIdx.x + i * PB] = m[i];
#pragma unroll
  for (int i = 0; i < PC; ++i) reinterpret_cast<u32x4*>(hcnt)[threadIdx.x + i * PB] = c[i];
}

// Lowest non-empty bin of hmass/hcnt[0, nbins) whose mass from the top
// (exclusive) is <= P; returns it and its exclusive mass above.
__device__ inline int crossing_bin(const unsigned long long* hmass, const unsigned int* hcnt, int nbins,
                                   unsigned long long P, unsigned long long* red, int* s_low,
                                   unsigned long long* s_above, unsigned long long* above) {
  const int tid = threadIdx.x;
  const int per = nbins / PB;
  const int hi_bin = nbins - 1 - tid * per;
  unsigned long long m = 0;
  for (int i = 0; i < per; ++i) m += hmass[hi_bin - i];
  if (tid == 0) *s_low = nbins;
  unsigned long long tot;
  const unsigned long long before = block_scan(m, red, &tot);   // ends with a barrier
  {
    unsigned long long acc = before;
    int best = nbins;
    for (int i = 0; i < per; ++i) {
      const int b = hi_bin - i;
      if (hcnt[b] && acc <= P) best = b;
      acc += hmass[b];
    }
    if (best < nbins) atomicMin(s_low, best);
  }
  __syncthreads();
  const int b = *s_low;
  if (b <= hi_bin && b > hi_bin - per) {
    unsigned long long acc = before;
    for (int i = 0; i < per && hi_bin - i != b; ++i) acc += hmass[hi_bin - i];
    *s_above = acc;
  }
  __syncthreads();
  *above = *s_above;
  return b;
}

constexpr int UNR = 16;   // loads per thread in flight in the strided passes

// Thread-strided pass over ids [i0, i1) with UNR loads issued before any use.
template <typename F>
__device__ inline void strided_pass(const float* src, int i0, int i1, F&& f) {
  for (int b = i0 + (int)threadIdx.x; b < i1; b += UNR * PB) {
    float v[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int i = b + u * PB;
      v[u] = i < i1 ? src[i] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int i = b + u * PB;
      if (i < i1) f(i, v[u]);
    }
  }
}

// Ordered sub-chunks: wave w owns ids [s0 + w*SEGW, s0 + (w+1)*SEGW) and
// walks them in 64-id steps (step e, lane l: id s0 + w*SEGW + 64e + l), so
// loads and stores are coalesced and (wave, step, lane) is ascending id order.
__device__ inline int seg_id(int s0, int e) { return s0 + (int)(threadIdx.x >> 6) * SEGW + 64 * e + (int)(threadIdx.x & 63); }

// z of this lane's ids of the sub-chunk at s0 (ids at or past i1 read as 0).
__device__ inline void load_run(const float* z, int s0, int i1, float (&v)[RPT]) {
#pragma unroll
  for (int e = 0; e < RPT; ++e) {
    const int i = seg_id(s0, e);
    v[e] = i < i1 ? z[i] : 0.f;
  }
}

__device__ inline unsigned long long lanemask_lt() { return (1ull << (threadIdx.x & 63)) - 1ull; }

// Ranks of the ties at the cut in a sub-chunk: on return tie0 is the number
// of ties before this wave's segment (given tie_run before the sub-chunk) and
// tie_run has advanced past the sub-chunk.
__device__ inline unsigned int wave_tie_base(const float (&v)[RPT], int s0, int i1, unsigned int cut,
                                             unsigned int* wtie, unsigned int& tie_run) {
  unsigned int c = 0;
#pragma unroll
  for (int e = 0; e < RPT; ++e) c += (unsigned int)__popcll(__ballot(seg_id(s0, e) < i1 && f2key(v[e]) == cut));
  if ((threadIdx.x & 63) == 0) wtie[threadIdx.x >> 6] = c;
  __syncthreads();
  unsigned int before = tie_run, tot = 0;
  for (int w = 0; w < NW; ++w) {
    if (w < (int)(threadIdx.x >> 6)) before += wtie[w];
    tot += wtie[w];
  }
  __syncthreads();
  tie_run += tot;
  return before;
}

// ---- pass 1: penalty, temperature, chunk max; clear the histogram ----
__global__ __launch_bounds__(PB) void pen_z_kernel(const PenaltyParams p, int nb) {
  __shared__ unsigned int bitmap[MAX_V / 32];
  __shared__ float red[NW];
  const int row = blockIdx.y, tid = threadIdx.x;
  const PenWs ws = carve(p.ws, p.rows);
  int i0, i1;
  chunk_of(p.V, nb, blockIdx.x, &i0, &i1);
  if (p.top_p < 1.0f) {   // this chunk's share of the row's histogram
    const int h0 = blockIdx.x * H1 / nb, h1 = (blockIdx.x + 1) * H1 / nb;
    for (int b = h0 + tid; b < h1; b += PB) {
      ws.hmass[row * H1 + b] = 0ull;
      ws.hcnt[row * H1 + b] = 0u;
    }
  }
  const int nwords = (i1 - i0 + 31) / 32;
  for (int w = tid; w < nwords; w += PB) bitmap[w] = 0u;
  __syncthreads();
  if (p.W > 0) {
    const int32_t* win = p.window + (int64_t)row * p.window_stride;
    constexpr int WB = 8;   // window ids per thread in flight
    for (int w0 = tid; w0 < p.W; w0 += PB * WB) {
      int id[WB];
#pragma unroll
      for (int u = 0; u < WB; ++u) id[u] = w0 + u * PB < p.W ? win[w0 + u * PB] : -1;
#pragma unroll
      for (int u = 0; u < WB; ++u)
        if (id[u] >= i0 && id[u] < i1) atomicOr(&bitmap[(id[u] - i0) >> 5], 1u << ((id[u] - i0) & 31));
    }
  }
  __syncthreads();
  const float* x = p.logits + (int64_t)row * p.V;
  float* z = p.logits_out + (int64_t)row * p.V;
  float mx = -INFINITY;
  strided_pass(x, i0, i1, [&](int i, float v) {
    if ((bitmap[(i - i0) >> 5] >> ((i - i0) & 31)) & 1u) v = v > 0.f ? v / p.penalty : v * p.penalty;
    v = v / p.temperature;
    z[i] = v;
    mx = fmaxf(mx, v);
  });
  mx = block_max(mx, red);
  if (tid == 0) ws.bmax[row * NBR_MAX + blockIdx.x] = mx;
}

// ---- pass 2: mass histogram and chunk mass ----
__global__ __launch_bounds__(PB) void pen_hist_kernel(const PenaltyParams p, int nb) {
  __shared__ unsigned long long hmass[H1];
  __shared__ unsigned int hcnt[H1];
  __shared__ unsigned long long red64[NW];
  __shared__ float redf[NW];
  const int row = blockIdx.y, tid = threadIdx.x;
  const PenWs ws = carve(p.ws, p.rows);
  int i0, i1;
  chunk_of(p.V, nb, blockIdx.x, &i0, &i1);
  for (int b = tid; b < H1; b += PB) {
    hmass[b] = 0ull;
    hcnt[b] = 0u;
  }
  const float zmax = row_max(ws, row, nb, redf);   // its barriers also order the clears
  const float* z = p.logits_out + (int64_t)row * p.V;
  unsigned long long zsum = 0;
  strided_pass(z, i0, i1, [&](int, float v) {
    const unsigned long long f = to_fix(__expf(v - zmax));
    const unsigned int b = f2key(v) >> (32 - H1_BITS);
    atomicAdd(&hmass[b], f);
    atomicAdd(&hcnt[b], 1u);
    zsum += f;
  });
  zsum = block_sum(zsum, red64);   // its barriers also retire the LDS atomics
  for (int b = tid; b < H1; b += PB) {
    const unsigned int c = hcnt[b];
    if (c) {
      atomicAdd(&ws.hmass[row * H1 + b], hmass[b]);
      atomicAdd(&ws.hcnt[row * H1 + b], c);
    }
  }
  if (tid == 0) ws.zs[row * NBR_MAX + blockIdx.x] = zsum;
}

// ---- pass 3: the crossing bin and the chunk's keys in it ----
__global__ __launch_bounds__(PB) void pen_cutbin_kernel(const PenaltyParams p, int nb) {
  __shared__ __attribute__((aligned(16))) unsigned long long hmass[H1];
  __shared__ __attribute__((aligned(16))) unsigned int hcnt[H1];
  __shared__ unsigned long long red64[NW];
  __shared__ int s_low;
  __shared__ unsigned long long s_above;
  __shared__ unsigned int s_n;
  const int row = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
  const PenWs ws = carve(p.ws, p.rows);
  int i0, i1;
  chunk_of(p.V, nb, blockIdx.x, &i0, &i1);
  const float* z = p.logits_out + (int64_t)row * p.V;
  float v[RPT];
  load_run(z, i0, i1, v);   // the first sub-chunk, in flight with the histogram
  load_hist(hmass, hcnt, ws, row);
  if (tid == 0) s_n = 0;
  const unsigned long long Z = row_mass(ws, row, nb, red64);
  const unsigned long long P = (unsigned long long)((double)p.top_p * (double)Z);
  unsigned long long above;
  const unsigned int bin = (unsigned int)crossing_bin(hmass, hcnt, H1, P, red64, &s_low, &s_above, &above);
  unsigned int* cand = ws.cand + (int64_t)row * p.V + i0;
  for (int s0 = i0; s0 < i1; s0 += SUBC) {
    if (s0 != i0) load_run(z, s0, i1, v);
#pragma unroll
    for (int e = 0; e < RPT; ++e) {
      const bool take = seg_id(s0, e) < i1 && (f2key(v[e]) >> (32 - H1_BITS)) == bin;
      const unsigned long long m = __ballot(take);
      if (m) {   // one LDS atomic per wave step with takers
        const int leader = __ffsll((long long)m) - 1;
        unsigned int base = 0;
        if (lane == leader) base = atomicAdd(&s_n, (unsigned int)__popcll(m));
        base = __shfl(base, leader);
        if (take) cand[base + (unsigned int)__popcll(m & lanemask_lt())] = f2key(v[e]);
      }
    }
  }
  __syncthreads();
  if (tid == 0) ws.ccnt[row * NBR_MAX + blockIdx.x] = s_n;
}

// The cut as every pass after the refinement sees it.
struct Cut {
  bool all_top, rank_ties;
  unsigned int cut, ties_kept;
  float zmax, ln_min_p;
};

// Keep decisions of one 64-id step (all lanes call it): `tie_i` counts the
// ties at the cut before the step (ids ascending) and advances past it.
__device__ inline bool keep_step(const Cut& c, float zv, bool valid, unsigned int& tie_i) {
  const unsigned int key = f2key(zv);
  bool top = c.all_top || key > c.cut;
  const bool tie = !c.all_top && valid && key == c.cut;
  const unsigned long long tm = __ballot(tie);
  if (tie) top = !c.rank_ties || tie_i + (unsigned int)__popcll(tm & lanemask_lt()) < c.ties_kept;
  tie_i += (unsigned int)__popcll(tm);
  return valid && top && (zv - c.zmax >= c.ln_min_p);
}

// ---- pass 4: exact cut, keep mask and the chunk's kept mass ----
__global__ __launch_bounds__(PB) void pen_keep_kernel(const PenaltyParams p, int nb) {
  __shared__ __attribute__((aligned(16))) unsigned long long hmass[H1];
  __shared__ __attribute__((aligned(16))) unsigned int hcnt[H1];
  __shared__ unsigned int cand_l[CAND_CAP];
  __shared__ unsigned long long red64[NW];
  __shared__ float redf[NW];
  __shared__ unsigned int redu[NW];
  __shared__ unsigned int seg_off[NBR_MAX + 1];
  __shared__ int s_low;
  __shared__ unsigned long long s_above;
  const int row = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
  const PenWs ws = carve(p.ws, p.rows);
  int i0, i1;
  chunk_of(p.V, nb, blockIdx.x, &i0, &i1);
  const float* z = p.logits_out + (int64_t)row * p.V;
  float v[RPT];
  load_run(z, i0, i1, v);   // the first sub-chunk, in flight with what follows
  Cut c;
  c.all_top = p.top_p >= 1.0f;
  c.ln_min_p = logf(p.min_p);   // -inf for min_p = 0
  c.cut = 0u;
  c.ties_kept = 0u;
  c.rank_ties = false;
  unsigned int tie_before = 0;   // ties at the cut in earlier chunks
  if (!c.all_top) {
    load_hist(hmass, hcnt, ws, row);
    if (tid < 64) {   // list offsets: one wave scans the chunks' list lengths
      const unsigned int cn = lane < nb ? ws.ccnt[row * NBR_MAX + lane] : 0u;
      unsigned int incl = cn;
      for (int off = 1; off < 64; off <<= 1) {
        const unsigned int y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
      }
      if (lane < nb) seg_off[lane] = incl - cn;
      if (lane == 63) seg_off[nb] = incl;
    }
  }
  c.zmax = row_max(ws, row, nb, redf);   // its barriers also publish the loads above
  if (!c.all_top) {
    unsigned long long P = (unsigned long long)((double)p.top_p * (double)row_mass(ws, row, nb, red64));
    const unsigned int n = seg_off[nb];
    const unsigned int* cand_g = ws.cand + (int64_t)row * p.V;
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
      int c0, c1;
      chunk_of(p.V, nb, b, &c0, &c1);
      return cand_g[c0 + (i - seg_off[b])];
    };
    const bool in_lds = n <= (unsigned int)CAND_CAP;
    if (in_lds) {
      constexpr int BATCH = 8;
      for (unsigned int b0 = tid; b0 < n; b0 += PB * BATCH) {
        unsigned int kv[BATCH];
#pragma unroll
        for (int u = 0; u < BATCH; ++u) kv[u] = b0 + u * PB < n ? key_at(b0 + u * PB) : 0u;
#pragma unroll
        for (int u = 0; u < BATCH; ++u)
          if (b0 + u * PB < n) cand_l[b0 + u * PB] = kv[u];
      }
    }
    __syncthreads();
    unsigned long long above;
    unsigned int prefix = (unsigned int)crossing_bin(hmass, hcnt, H1, P, red64, &s_low, &s_above, &above);
    P -= above;
    int shift = 32 - H1_BITS;
    unsigned int cut_count = 0;
    for (int pass = 0; pass < 2; ++pass) {
      constexpr int nbins = 1 << 10;
      const int new_shift = shift - 10;
      __syncthreads();
      for (int b = tid; b < nbins; b += PB) {
        hmass[b] = 0ull;
        hcnt[b] = 0u;
      }
      __syncthreads();
      for (unsigned int i = tid; i < n; i += PB) {
        const unsigned int key = in_lds ? cand_l[i] : key_at(i);
        if ((key >> shift) == prefix) {
          const unsigned int b = (key >> new_shift) & (nbins - 1);
          atomicAdd(&hmass[b], to_fix(__expf(key2f(key) - c.zmax)));
          atomicAdd(&hcnt[b], 1u);
        }
      }
      __syncthreads();
      const int b = crossing_bin(hmass, hcnt, nbins, P, red64, &s_low, &s_above, &above);
      P -= above;
      if (pass == 1) cut_count = hcnt[b];
      prefix = (prefix << 10) | (unsigned int)b;
      shift = new_shift;
    }
    c.cut = prefix;
    const unsigned long long ecut = to_fix(__expf(key2f(c.cut) - c.zmax));
    // ties at the cut: the t-th (0-based, ids ascending) has mass before it = above + t * ecut
    const unsigned long long nt = ecut ? P / ecut + 1ull : (unsigned long long)cut_count;
    c.ties_kept = nt < cut_count ? (unsigned int)nt : cut_count;
    c.rank_ties = c.ties_kept < cut_count;
    if (c.rank_ties) {   // ties in earlier chunks: their listed keys equal to the cut
      unsigned int t = 0;
      for (unsigned int i = tid; i < seg_off[blockIdx.x]; i += PB) t += (in_lds ? cand_l[i] : key_at(i)) == c.cut;
      tie_before = block_sum(t, redu);
    }
    if (tid == 0) {
      ws.tie0[row * NBR_MAX + blockIdx.x] = tie_before;
      if (blockIdx.x == 0) {
        ws.cut[row * 4 + 0] = c.cut;
        ws.cut[row * 4 + 1] = c.ties_kept;
        ws.cut[row * 4 + 2] = cut_count;
      }
    }
  }
  // keep mask and kept mass; ties are ranked by id (per-wave counts, then ballots)
  float wsum = 0.f;
  unsigned int tie_run = tie_before;
  for (int s0 = i0; s0 < i1; s0 += SUBC) {
    if (s0 != i0) load_run(z, s0, i1, v);
    unsigned int tie_i = c.rank_ties ? wave_tie_base(v, s0, i1, c.cut, redu, tie_run) : 0u;
#pragma unroll
    for (int e = 0; e < RPT; ++e) {
      const int i = seg_id(s0, e);
      const bool valid = i < i1;
      const bool k = keep_step(c, v[e], valid, tie_i);
      if (valid && p.keep) p.keep[(int64_t)row * p.V + i] = (uint8_t)k;
      wsum += k ? __expf(v[e] - c.zmax) : 0.f;
    }
  }
  wsum = block_sum(wsum, redf);
  if (tid == 0) ws.km[row * NBR_MAX + blockIdx.x] = wsum;
}

// ---- pass 5: probabilities and the token ----
__global__ __launch_bounds__(PB) void pen_probs_kernel(const PenaltyParams p, int nb) {
  __shared__ float redf[NW];
  __shared__ unsigned int redu[NW];
  __shared__ float s_km[NBR_MAX];
  __shared__ int s_tok, s_last;
  const int row = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const PenWs ws = carve(p.ws, p.rows);
  int i0, i1;
  chunk_of(p.V, nb, blockIdx.x, &i0, &i1);
  const float* z = p.logits_out + (int64_t)row * p.V;
  float v[RPT];
  load_run(z, i0, i1, v);   // the first sub-chunk, in flight with what follows
  Cut c;
  c.all_top = p.top_p >= 1.0f;
  c.ln_min_p = logf(p.min_p);
  c.cut = c.all_top ? 0u : ws.cut[row * 4 + 0];
  c.ties_kept = c.all_top ? 0u : ws.cut[row * 4 + 1];
  c.rank_ties = !c.all_top && c.ties_kept < ws.cut[row * 4 + 2];
  unsigned int tie_run = c.rank_ties ? ws.tie0[row * NBR_MAX + blockIdx.x] : 0u;
  if (tid < nb) s_km[tid] = ws.km[row * NBR_MAX + tid];
  if (tid == 0) {
    s_tok = INT_MAX;
    s_last = -1;
  }
  c.zmax = row_max(ws, row, nb, redf);   // its barriers also publish s_km
  float S = 0.f, wbase = 0.f;   // row kept mass, kept mass of earlier chunks (fixed order)
  int last_chunk = -1;          // last chunk with kept mass
  for (int b = 0; b < nb; ++b) {
    if (b < (int)blockIdx.x) wbase += s_km[b];
    S += s_km[b];
    if (s_km[b] > 0.f) last_chunk = b;
  }
  const float inv = 1.0f / S;
  const float target = p.u ? p.u[row] * S : 0.f;
  const float my = s_km[blockIdx.x];
  // the chunk whose kept-mass range holds the target searches it; if rounding
  // put the target at or past the total, the last kept id is the token
  const bool mine = p.token && ((target >= wbase && target < wbase + my) ||
                                (target >= S && (int)blockIdx.x == last_chunk));
  float run = wbase;
  bool found = false;
  for (int s0 = i0; s0 < i1; s0 += SUBC) {
    if (s0 != i0) load_run(z, s0, i1, v);
    unsigned int tie_i = c.rank_ties ? wave_tie_base(v, s0, i1, c.cut, redu, tie_run) : 0u;
    float ev[RPT];
    float esum = 0.f;
    int last_kept = -1;
#pragma unroll
    for (int e = 0; e < RPT; ++e) {
      const int i = seg_id(s0, e);
      const bool valid = i < i1;
      const bool k = keep_step(c, v[e], valid, tie_i);
      ev[e] = k ? __expf(v[e] - c.zmax) : 0.f;
      if (valid && p.probs) p.probs[(int64_t)row * p.V + i] = ev[e] * inv;
      esum += ev[e];
      if (k) last_kept = i;
    }
    if (mine && !found) {   // block-uniform: inverse CDF over this sub-chunk, ids ascending
      for (int m = 32; m >= 1; m >>= 1) esum += __shfl_xor(esum, m);
      if (lane == 0) redf[wave] = esum;
      __syncthreads();
      float acc = run, tot = 0.f;
      for (int w = 0; w < NW; ++w) {
        if (w < wave) acc += redf[w];
        tot += redf[w];
      }
      __syncthreads();
      int hit = INT_MAX;
#pragma unroll
      for (int e = 0; e < RPT; ++e) {
        float incl = ev[e];   // inclusive prefix over the step's lanes
        for (int off = 1; off < 64; off <<= 1) {
          const float y = __shfl_up(incl, off);
          if (lane >= off) incl += y;
        }
        const unsigned long long h = __ballot(ev[e] > 0.f && acc + incl > target);
        if (h && hit == INT_MAX) hit = seg_id(s0, e) - lane + __ffsll((long long)h) - 1;
        acc += __shfl(incl, 63);
      }
      if (lane == 0 && hit != INT_MAX) atomicMin(&s_tok, hit);
      if (last_kept >= 0) atomicMax(&s_last, last_kept);
      __syncthreads();
      run += tot;
      found = s_tok != INT_MAX;
      __syncthreads();
    }
  }
  if (mine && tid == 0) p.token[row] = s_tok != INT_MAX ? s_tok : s_last;
}

}  // namespace

int penalty_blocks_per_row(int32_t rows, int32_t V) {
  int nb = (256 + rows - 1) / rows;         // about one workgroup per compute unit over all rows
  const int by_ids = (V + 4095) / 4096;     // at least 4096 ids per workgroup
  if (nb > by_ids) nb = by_ids;
  if (nb > NBR_MAX) nb = NBR_MAX;
  if (nb < 1) nb = 1;
  return nb;
}

size_t penalty_workspace_bytes(int32_t rows, int32_t V) { return pen_ws_bytes(rows, V); }

hipError_t launch_penalty(const PenaltyParams& p, hipStream_t stream) {
  const int nb = penalty_blocks_per_row(p.rows, p.V);
  const dim3 grid(nb, p.rows);
  hipLaunchKernelGGL(pen_z_kernel, grid, dim3(PB), 0, stream, p, nb);
  if (p.top_p < 1.0f) {
    hipLaunchKernelGGL(pen_hist_kernel, grid, dim3(PB), 0, stream, p, nb);
    hipLaunchKernelGGL(pen_cutbin_kernel, grid, dim3(PB), 0, stream, p, nb);
  }
  hipLaunchKernelGGL(pen_keep_kernel, grid, dim3(PB), 0, stream, p, nb);
  if (p.probs || p.token) hipLaunchKernelGGL(pen_probs_kernel, grid, dim3(PB), 0, stream, p, nb);
  return hipGetLastError();
}

}  // namespace ts
