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
// Both filters keep a prefix of the (p desc, id asc) order, so the kept set
// is the shorter of the two prefixes, and every token ordered before a min-p
// token is itself a min-p token: the top-p masses inside the min-p set need
// nothing outside it. On peaked rows the min-p set is small (a few hundred
// ids of a 128K vocabulary at min_p = 0.05), so the pass decides on it alone
// whenever it fits, and runs a radix select over the whole row only when it
// does not (min_p near 0, flat rows).
//
// Two launches; every row is split into nb chunks of ids, one 512-thread
// workgroup each, so a few rows still spread over the whole chip:
//   1. z    window ids of the chunk -> LDS bitmap (set semantics makes
//           duplicates harmless); penalty and temperature -> logits_out; the
//           chunk's max m_b and sum of exp(z - m_b), merged in a fixed order;
//           the chunk's candidates z - m_b >= ln(min_p) (a superset of its
//           min-p members, as m_b <= max z), listed as sort keys (z
//           descending, id ascending), at most CAP_B per chunk.
//   2. out  every workgroup of a row takes the same decision: row max and mass
//           Z from the chunk partials; if no list overflowed, the min-p set S
//           from the lists (at most SCAP); if the mass of S less its lightest
//           member is within top_p * Z, all of S is kept, else S is sorted in
//           LDS and cut by exclusive prefix mass. Otherwise a radix select over
//           the whole row (a 12-bit and two 10-bit digits of the key, mass
//           histograms) gives the top-p cut key and how many of its ties (ids
//           ascending) stay. The token, when the kept set is listed, comes
//           from the one workgroup whose chunk holds the crossing of u times
//           the kept mass (else from an ordered scan of the row by the first
//           workgroup); then the chunk's keep mask and renormalised
//           probabilities.
// Eta-sampling variant (Appendix D.1: the pool is the tokens whose
// probability reaches eta, built from the entropy and constants alpha and
// epsilon): eta = min(epsilon, alpha exp(-H)), H in nats, and the most
// probable token always stays, so the pool is p_i >= min(eta, max p), i.e.
// z_i - max z >= ln(min(1, eta Z)). Three launches, same grid:
//   1. z     as above, plus each chunk's sum of exp(z - m_b) z (no lists: the
//            threshold is not known yet);
//   2. mass  every workgroup merges the partials into H = ln Z + max z -
//            (sum e z) / Z (double) and the threshold, then stores its
//            chunk's kept mass and last kept id;
//   3. out   the row's kept mass W and the mass below the chunk (exact
//            fixed-point sums), the chunk's keep mask and probabilities, and
//            the token from the one workgroup whose chunk holds the crossing
//            of u W (an ordered scan of that chunk only).
// The mass of one token is exp(z - max z) in fp32 taken to 2^-40 fixed point,
// so every prefix mass is an exact integer sum, whatever the summation order.
// The penalty and the temperature are applied as products with their fp32
// reciprocals (within two roundings of the quotients).
#include "ts_device.h"
#include "ts_internal.h"

#include <climits>
#include <cmath>

namespace ts {
namespace {

constexpr int PB = 512;                 // threads per workgroup
constexpr int NW = PB / 64;
constexpr int NBR_MAX = 64;             // workgroups per row
constexpr int H1_BITS = 12;
constexpr int H1 = 1 << H1_BITS;        // bins of the first radix digit
constexpr int H2 = 1 << 10;             // bins of the second and third digits
constexpr int MAX_V = 262144;
constexpr int RPT = 16;                 // 64-id steps per wave in an ordered sub-chunk
constexpr int SEGW = 64 * RPT;          // ids per wave segment of a sub-chunk
constexpr int SUBC = PB * RPT;          // ids per ordered sub-chunk (NW segments, ascending)
constexpr int CAP_B = 1024;             // candidates listed per chunk
constexpr int SCAP = 4096;              // largest min-p set decided in LDS
constexpr int UNR = 16;                 // loads per thread in flight in the strided passes
constexpr int ZR = 32;                  // ids per thread held in registers in pass 1
constexpr float FIX_SCALE = 1099511627776.0f;  // 2^40
static_assert(SCAP == H1, "the sorted list and the first-digit mass histogram share LDS");
static_assert(H2 % PB == 0 && H1 % PB == 0, "bins split evenly over the threads");

__device__ inline float key2f(unsigned int k) {
  const unsigned int u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}
__device__ inline u64 to_fix(float e) { return (u64)(e * FIX_SCALE); }

// Sort key: ascending order is z descending, then id ascending.
__device__ inline u64 sort_key(float z, int id) { return ((u64)(~f2key(z)) << 32) | (unsigned int)id; }
__device__ inline unsigned int sk_key(u64 s) { return ~(unsigned int)(s >> 32); }
__device__ inline int sk_id(u64 s) { return (int)(unsigned int)s; }

__host__ __device__ inline size_t round256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

int penalty_blocks_per_row(int32_t rows, int32_t V) {
  int nb = 256 / rows;                      // about one workgroup per compute unit over all rows,
  const int by_regs = (V + ZR * PB - 1) / (ZR * PB);   // but chunks small enough for the register path
  if (nb < by_regs) nb = by_regs;
  const int by_ids = (V + 4095) / 4096;     // at least 4096 ids per workgroup
  if (nb > by_ids) nb = by_ids;
  if (nb > NBR_MAX) nb = NBR_MAX;
  if (nb < 1) nb = 1;
  return nb;
}

namespace {

// Workspace (256-byte aligned pieces):
//   pm   [rows][NBR_MAX] f32   chunk max of z
//   ps   [rows][NBR_MAX] f32   chunk sum of exp(z - chunk max)
//   pc   [rows][NBR_MAX] u32   chunk candidates (> CAP_B: the list overflowed)
//   pz   [rows][NBR_MAX] f32   chunk sum of exp(z - chunk max) * z (eta mode)
//   pw   [rows][NBR_MAX] u64   chunk kept mass, fixed point (eta mode)
//   pl   [rows][NBR_MAX] i32   chunk's last kept id, -1 if none (eta mode)
//   cand [rows][nb][CAP_B] u64 candidate sort keys
struct PenWs {
  float* pm;
  float* ps;
  unsigned int* pc;
  float* pz;
  u64* pw;
  int* pl;
  u64* cand;
};

__host__ __device__ inline PenWs carve(void* base, int rows) {
  char* w = static_cast<char*>(base);
  PenWs s;
  s.pm = reinterpret_cast<float*>(w);
  w += round256((size_t)rows * NBR_MAX * 4);
  s.ps = reinterpret_cast<float*>(w);
  w += round256((size_t)rows * NBR_MAX * 4);
  s.pc = reinterpret_cast<unsigned int*>(w);
  w += round256((size_t)rows * NBR_MAX * 4);
  s.pz = reinterpret_cast<float*>(w);
  w += round256((size_t)rows * NBR_MAX * 4);
  s.pw = reinterpret_cast<u64*>(w);
  w += round256((size_t)rows * NBR_MAX * 8);
  s.pl = reinterpret_cast<int*>(w);
  w += round256((size_t)rows * NBR_MAX * 4);
  s.cand = reinterpret_cast<u64*>(w);
  return s;
}

size_t pen_ws_bytes(int rows, int V) {
  const int nb = penalty_blocks_per_row(rows, V);
  return 5 * round256((size_t)rows * NBR_MAX * 4) + round256((size_t)rows * NBR_MAX * 8) +
         round256((size_t)rows * nb * CAP_B * 8);
}

// Chunk b of nb over ids [0, V): a multiple of 64 ids.
__device__ inline void chunk_of(int V, int nb, int b, int* i0, int* i1) {
  const int chunk = ((V + nb - 1) / nb + 63) / 64 * 64;
  *i0 = min(b * chunk, V);
  *i1 = min(*i0 + chunk, V);
}



// ---- block reductions (fixed order: results do not depend on timing) ----
__device__ inline float block_max(float x, float* red) {
  x = wave_reduce(x, OpMax());
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  bar();
  float r = red[0];
  for (int w = 1; w < NW; ++w) r = fmaxf(r, red[w]);
  bar();
  return r;
}

template <typename T>
__device__ inline T block_sum(T x, T* red) {
  x = wave_reduce(x, OpAdd());
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  bar();
  T r = red[0];
  for (int w = 1; w < NW; ++w) r += red[w];
  bar();
  return r;
}

// Exclusive prefix over threads (thread order); *total gets the sum.
template <typename T>
__device__ inline T block_scan(T x, T* red, T* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const T incl = wave_incl_scan(x);
  if (lane == 63) red[wave] = incl;
  bar();
  T pre = 0, tot = 0;
  for (int w = 0; w < NW; ++w) {
    if (w < wave) pre += red[w];
    tot += red[w];
  }
  bar();
  *total = tot;
  return pre + incl - x;
}

// Lowest non-empty bin of hmass/hcnt[0, nbins) whose mass from the top
// (exclusive) is <= P; returns it and its exclusive mass above.
__device__ inline int crossing_bin(const u64* hmass, const unsigned int* hcnt, int nbins, u64 P, u64* red,
                                   int* s_low, u64* s_above, u64* above) {
  const int tid = threadIdx.x;
  const int per = nbins / PB;
  const int hi_bin = nbins - 1 - tid * per;
  u64 m = 0;
  for (int i = 0; i < per; ++i) m += hmass[hi_bin - i];
  if (tid == 0) *s_low = nbins;
  u64 tot;
  const u64 before = block_scan(m, red, &tot);   // ends with a barrier
  {
    u64 acc = before;
    int best = nbins;
    for (int i = 0; i < per; ++i) {
      const int b = hi_bin - i;
      if (hcnt[b] && acc <= P) best = b;
      acc += hmass[b];
    }
    if (best < nbins) atomicMin(s_low, best);
  }
  bar();
  const int b = *s_low;
  if (b <= hi_bin && b > hi_bin - per) {
    u64 acc = before;
    for (int i = 0; i < per && hi_bin - i != b; ++i) acc += hmass[hi_bin - i];
    *s_above = acc;
  }
  bar();
  *above = *s_above;
  return b;
}

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

// Ranks of the ties at the cut in a sub-chunk: returns the number of ties
// before this wave's segment (given tie_run before the sub-chunk) and
// advances tie_run past the sub-chunk.
__device__ inline unsigned int wave_tie_base(const float (&v)[RPT], int s0, int i1, unsigned int cut,
                                             unsigned int* wtie, unsigned int& tie_run) {
  unsigned int c = 0;
#pragma unroll
  for (int e = 0; e < RPT; ++e) c += (unsigned int)__popcll(__ballot(seg_id(s0, e) < i1 && f2key(v[e]) == cut));
  if ((threadIdx.x & 63) == 0) wtie[threadIdx.x >> 6] = c;
  bar();
  unsigned int before = tie_run, tot = 0;
  for (int w = 0; w < NW; ++w) {
    if (w < (int)(threadIdx.x >> 6)) before += wtie[w];
    tot += wtie[w];
  }
  bar();
  tie_run += tot;
  return before;
}

// The kept set as every workgroup of the row sees it: keys above `cut` and
// the first ties_kept ids with key == cut (all of them unless rank_ties), or
// every key when all_top; then the min-p test.
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
  const u64 tm = __ballot(tie);
  if (tie) top = !c.rank_ties || tie_i + (unsigned int)__popcll(tm & lanemask_lt()) < c.ties_kept;
  tie_i += (unsigned int)__popcll(tm);
  return valid && top && (zv - c.zmax >= c.ln_min_p);
}

// Ascending in-place bitonic sort of s[0, n), n a power of two, by the whole
// workgroup; ends with a barrier.
__device__ inline void bitonic_sort(u64* s, int n) {
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n; i += PB) {
        const int pr = i ^ j;
        if (pr > i) {
          const u64 a = s[i], b = s[pr];
          const bool up = (i & k) == 0;
          if ((a > b) == up) {
            s[i] = b;
            s[pr] = a;
          }
        }
      }
      bar();
    }
  }
}

// Appends the values of the taking lanes of N wave steps to an LDS-counted
// list with one LDS atomic per wave (step order, then lane order);
// put(step, slot) stores one value. The counter counts every taker.
template <int N, typename F>
__device__ inline void wave_append(const bool (&take)[N], unsigned int* counter, F&& put) {
  u64 bm[N];
  unsigned int tot = 0;
#pragma unroll
  for (int r = 0; r < N; ++r) {
    bm[r] = __ballot(take[r]);
    tot += (unsigned int)__popcll(bm[r]);
  }
  if (tot == 0u) return;   // wave-uniform
  unsigned int base = 0;
  if ((threadIdx.x & 63) == 0) base = atomicAdd(counter, tot);
  base = __builtin_amdgcn_readfirstlane(base);
#pragma unroll
  for (int r = 0; r < N; ++r) {
    if (take[r]) put(r, base + (unsigned int)__popcll(bm[r] & lanemask_lt()));
    base += (unsigned int)__popcll(bm[r]);
  }
}

__device__ inline int pow2_at_least(int n) {
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}

// ---- pass 1: penalty, temperature, chunk partials and min-p candidates ----
// Chunks of up to ZR * PB ids stay in registers (one read of the logits, the
// window ids in flight with them; 16-byte accesses of 4 ids when the rows are
// 16-byte aligned); larger ones (few rows) take a strided loop with an online
// sum and re-read their own z for the candidates.
typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(PB) void pen_z_kernel(const PenaltyParams p, int nb) {
  __shared__ unsigned int bitmap[MAX_V / 32];
  __shared__ float redf[NW];
  __shared__ unsigned int s_n;
  const int row = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
  const PenWs ws = carve(p.ws, p.rows);
  int i0, i1;
  chunk_of(p.V, nb, blockIdx.x, &i0, &i1);
  const float* x = p.logits + (int64_t)row * p.V;
  float* z = p.logits_out + (int64_t)row * p.V;
  const bool in_regs = i1 - i0 <= ZR * PB;
  // 4 ids per access: chunk bounds are then multiples of 4 (i0 of 64, V of 4)
  const bool vec = in_regs && (p.V & 3) == 0 &&
                   ((reinterpret_cast<uintptr_t>(p.logits) | reinterpret_cast<uintptr_t>(p.logits_out)) & 15) == 0;
  // id of register slot u
  auto slot_id = [&](int u) { return vec ? i0 + 4 * (tid + (u >> 2) * PB) + (u & 3) : i0 + tid + u * PB; };
  float v[ZR];
  if (vec) {
#pragma unroll
    for (int q = 0; q < ZR / 4; ++q) {
      const int g = i0 + 4 * (tid + q * PB);
      const f32x4 t = g < i1 ? *reinterpret_cast<const f32x4*>(x + g) : f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
      for (int c = 0; c < 4; ++c) v[4 * q + c] = t[c];
    }
  } else if (in_regs) {
#pragma unroll
    for (int u = 0; u < ZR; ++u) {
      const int i = slot_id(u);
      v[u] = i < i1 ? x[i] : -INFINITY;
    }
  }
  constexpr int WB = 4;   // window ids per thread loaded with the logits
  const int32_t* win = p.window + (int64_t)row * p.window_stride;
  int wid[WB];
#pragma unroll
  for (int u = 0; u < WB; ++u) wid[u] = tid + u * PB < p.W ? win[tid + u * PB] : -1;
  const int nwords = (i1 - i0 + 31) / 32;
  for (int w = tid; w < nwords; w += PB) bitmap[w] = 0u;
  if (tid == 0) s_n = 0u;
  bar();
  auto mark = [&](int id) {
    if (id >= i0 && id < i1) atomicOr(&bitmap[(id - i0) >> 5], 1u << ((id - i0) & 31));
  };
#pragma unroll
  for (int u = 0; u < WB; ++u) mark(wid[u]);
  for (int j = tid + WB * PB; j < p.W; j += PB) mark(win[j]);
  bar();
  // x / penalty or x * penalty on window ids, then / temperature, by reciprocals
  const float inv_pen = 1.0f / p.penalty, inv_t = p.inv_temperature;
  auto penalised = [&](bool hit, float w) {
    w = hit ? (w > 0.f ? w * inv_pen : w * p.penalty) : w;
    return w * inv_t;
  };
  auto hit_at = [&](int i) { return ((bitmap[(i - i0) >> 5] >> ((i - i0) & 31)) & 1u) != 0u; };
  float mb, sb;
  if (in_regs) {
    // the slots' bitmap words first (all LDS reads in flight), then branch-free
    // arithmetic; slots past the chunk hold -inf and stay -inf
    unsigned int pw[ZR];
#pragma unroll
    for (int u = 0; u < ZR; ++u) {
      const int o = slot_id(u) - i0;   // < ZR * PB: inside the bitmap
      pw[u] = bitmap[o >> 5] >> (o & 31);
    }
    float m = -INFINITY;
#pragma unroll
    for (int u = 0; u < ZR; ++u) {
      v[u] = penalised((pw[u] & 1u) != 0u, v[u]);
      m = fmaxf(m, v[u]);
    }
    if (vec) {
#pragma unroll
      for (int q = 0; q < ZR / 4; ++q) {
        const int g = i0 + 4 * (tid + q * PB);
        if (g < i1) *reinterpret_cast<f32x4*>(z + g) = f32x4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
      }
    } else {
#pragma unroll
      for (int u = 0; u < ZR; ++u) {
        const int i = slot_id(u);
        if (i < i1) z[i] = v[u];
      }
    }
    mb = block_max(m, redf);
    float s = 0.f;
#pragma unroll
    for (int u = 0; u < ZR; ++u) s += v[u] > -INFINITY ? __expf(v[u] - mb) : 0.f;   // -inf past i1
    sb = block_sum(s, redf);
  } else {
    // running max of this thread's z and sum of exp(z - running max)
    float m = -INFINITY, s = 0.f;
    strided_pass(x, i0, i1, [&](int i, float w) {
      w = penalised(hit_at(i), w);
      z[i] = w;
      if (w > m) {
        s = s * __expf(m - w) + 1.f;
        m = w;
      } else if (w > -INFINITY) {
        s += __expf(w - m);
      }
    });
    mb = block_max(m, redf);
    sb = block_sum(m > -INFINITY ? s * __expf(m - mb) : 0.f, redf);
  }
  // eta mode: the chunk's sum of exp(z - mb) * z (the entropy's numerator)
  float szb = 0.f;
  if (p.eta_mode) {
    float sz = 0.f;
    if (in_regs) {
#pragma unroll
      for (int u = 0; u < ZR; ++u) sz += v[u] > -INFINITY ? __expf(v[u] - mb) * v[u] : 0.f;
    } else {
      for (int i = i0 + tid; i < i1; i += PB) {   // the z this thread wrote above
        const float w = z[i];
        sz += w > -INFINITY ? __expf(w - mb) * w : 0.f;
      }
    }
    szb = block_sum(sz, redf);
  }
  // candidates z - mb >= ln(min_p), listed by one LDS atomic per wave step with takers
  // (eta mode lists nothing: its threshold is known only in pass 2)
  const float ln_min_p = logf(p.min_p);   // -inf for min_p = 0
  const bool listed = !p.eta_mode && !(ln_min_p == -INFINITY && i1 - i0 > CAP_B);
  u64* out = ws.cand + ((int64_t)row * nb + blockIdx.x) * CAP_B;
  auto list_step = [&](int i, float w) {   // all lanes of the wave call it
    const bool take = i < i1 && w - mb >= ln_min_p;
    const u64 bm = __ballot(take);
    if (bm) {
      const int leader = __ffsll((long long)bm) - 1;
      unsigned int base = 0;
      if (lane == leader) base = atomicAdd(&s_n, (unsigned int)__popcll(bm));
      base = lane_value(base, leader);
      const unsigned int slot = base + (unsigned int)__popcll(bm & lanemask_lt());
      if (take && slot < (unsigned int)CAP_B) out[slot] = sort_key(w, i);
    }
  };
  if (listed) {
    if (in_regs) {
      bool take[ZR];
#pragma unroll
      for (int u = 0; u < ZR; ++u) take[u] = slot_id(u) < i1 && v[u] - mb >= ln_min_p;
      wave_append(take, &s_n, [&](int u, unsigned int slot) {
        if (slot < (unsigned int)CAP_B) out[slot] = sort_key(v[u], slot_id(u));
      });
    } else {
      // every thread re-reads the z it wrote above (same ids)
      for (int b = i0 + tid; b < i1; b += UNR * PB) {
        float w[UNR];
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
          const int i = b + u * PB;
          w[u] = i < i1 ? z[i] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < UNR; ++u) list_step(b + u * PB, w[u]);
      }
    }
  }
  bar();
  if (tid == 0) {
    ws.pm[row * NBR_MAX + blockIdx.x] = mb;
    ws.ps[row * NBR_MAX + blockIdx.x] = sb;
    ws.pc[row * NBR_MAX + blockIdx.x] = listed ? s_n : 0xffffffffu;
    ws.pz[row * NBR_MAX + blockIdx.x] = szb;
  }
}

// Ordered scan of ids [lo, hi) by the whole workgroup: the smallest id whose
// kept mass, counted from `run` (the kept mass below lo) and inclusive,
// exceeds target (INT_MAX if none), and in *last_out the last kept id of the
// scanned range (-1 if none). Sub-chunks of PB * RPT ids; thread t holds the
// RPT consecutive ids from s0 + t * RPT, so one block scan of the threads'
// kept masses (and, when the cut ranks its ties, one of their tie counts)
// puts the crossing inside one thread, which walks its ids. Stops at the
// sub-chunk that holds the crossing. Scratch: red64[NW], redu[NW], two LDS ints.
__device__ inline int ordered_token(const float* z, int lo, int hi, u64 run, u64 target, const Cut& c, u64* red64,
                                    unsigned int* redu, int* s_tok, int* s_lastkept, int* last_out) {
  const int tid = threadIdx.x;
  if (tid == 0) {
    *s_tok = INT_MAX;
    *s_lastkept = -1;
  }
  bar();
  unsigned int tie_run = 0;   // ties at the cut below the sub-chunk
  for (int s0 = lo; s0 < hi; s0 += SUBC) {
    const int j0 = s0 + tid * RPT;
    float v[RPT];
#pragma unroll
    for (int e = 0; e < RPT; ++e) v[e] = z[min(j0 + e, hi - 1)];   // ids past hi are invalid below
    unsigned int tie_i = 0;
    if (c.rank_ties) {   // workgroup-uniform
      unsigned int nt = 0;
#pragma unroll
      for (int e = 0; e < RPT; ++e) nt += (j0 + e < hi && f2key(v[e]) == c.cut) ? 1u : 0u;
      unsigned int tot_t;
      tie_i = tie_run + block_scan(nt, redu, &tot_t);
      tie_run += tot_t;
    }
    u64 ev[RPT];
    u64 sum = 0;
    int last = -1;
#pragma unroll
    for (int e = 0; e < RPT; ++e) {
      const bool valid = j0 + e < hi;
      const unsigned int key = f2key(v[e]);
      bool top = c.all_top || key > c.cut;
      if (!c.all_top && valid && key == c.cut) {   // ties ranked by id
        top = !c.rank_ties || tie_i < c.ties_kept;
        ++tie_i;
      }
      const bool k = valid && top && (v[e] - c.zmax >= c.ln_min_p);
      ev[e] = k ? to_fix(__expf(v[e] - c.zmax)) : 0ull;
      sum += ev[e];
      if (k) last = j0 + e;
    }
    u64 tot;
    const u64 excl = run + block_scan(sum, red64, &tot);
    if (sum > 0ull && excl <= target && target < excl + sum) {   // one thread at most
      u64 acc = excl;
      int hit = INT_MAX;
#pragma unroll
      for (int e = 0; e < RPT; ++e) {
        acc += ev[e];
        if (hit == INT_MAX && ev[e] > 0ull && acc > target) hit = j0 + e;
      }
      *s_tok = hit;
    }
    if (last >= 0) atomicMax(s_lastkept, last);
    bar();
    run += tot;
    const bool found = *s_tok != INT_MAX;
    bar();
    if (found) break;
  }
  *last_out = *s_lastkept;
  return *s_tok;
}

// ---- pass 2: the row's cut, keep mask, probabilities and token ----
constexpr int SPEC_R = 8;   // list entries per thread loaded together with the partials

__global__ __launch_bounds__(PB) void pen_out_kernel(const PenaltyParams p, int nb) {
  // the min-p set's sort keys, or the first-digit mass histogram of the radix select
  __shared__ __attribute__((aligned(16))) u64 list[SCAP];
  // counts of the radix select; the chunk's kept-id bitmap or the members' masses afterwards
  __shared__ __attribute__((aligned(16))) unsigned int hcnt[H1];
  __shared__ unsigned int hbefore[H2];
  __shared__ u64 red64[NW], red64b[NW];
  __shared__ unsigned int redu[NW];
  __shared__ unsigned int s_cnt[NBR_MAX];
  __shared__ float s_zmax;
  __shared__ double s_Z;
  __shared__ int s_over, s_low, s_k, s_first, s_last, s_tok, s_lastkept;
  __shared__ unsigned int s_n;
  __shared__ u64 s_above, s_w;
  const int row = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const PenWs ws = carve(p.ws, p.rows);
  const int V = p.V;
  int i0, i1;
  chunk_of(V, nb, blockIdx.x, &i0, &i1);
  const float* z = p.logits_out + (int64_t)row * V;

  // the first `per` entries of every list, in flight with the partials (entries
  // past a list's count are read but not used)
  const int per = min(CAP_B, SPEC_R * PB / nb);
  const u64* cand = ws.cand + (int64_t)row * nb * CAP_B;
  u64 spec[SPEC_R];
#pragma unroll
  for (int r = 0; r < SPEC_R; ++r) {
    const int idx = tid + r * PB, b = idx / per;
    spec[r] = b < nb ? cand[(int64_t)b * CAP_B + (idx - b * per)] : 0ull;
  }
  // row max, row mass Z (chunk sums rescaled, fixed order), list counts: one wave
  if (tid < 64) {
    const float mb = lane < nb ? ws.pm[row * NBR_MAX + lane] : -INFINITY;
    const float sb = lane < nb ? ws.ps[row * NBR_MAX + lane] : 0.f;
    const unsigned int cb = lane < nb ? ws.pc[row * NBR_MAX + lane] : 0u;
    const float zm = wave_reduce(mb, OpMax());
    const double sc = mb > -INFINITY ? (double)__expf(mb - zm) : 0.0;
    const double t = wave_reduce((double)sb * sc, OpAdd());
    const bool over = cb > (unsigned int)CAP_B;
    if (lane < nb) s_cnt[lane] = over ? 0u : cb;
    const u64 ob = __ballot(over);
    if (lane == 0) {
      s_zmax = zm;
      s_Z = t;
      s_over = ob != 0ull;
      s_n = 0u;
    }
  }
  bar();
  Cut c;
  c.zmax = s_zmax;
  c.ln_min_p = logf(p.min_p);   // -inf for min_p = 0
  c.all_top = p.top_p >= 1.0f;
  c.cut = 0u;
  c.ties_kept = 0u;
  c.rank_ties = false;
  const double Zfix = s_Z * (double)FIX_SCALE;
  const u64 P = c.all_top ? ~0ull : (u64)((double)p.top_p * Zfix);   // top-p mass bound, fixed point
  unsigned int tie_before = 0;   // ties at the cut with ids below the chunk
  u64 W = 0;                     // kept mass, fixed point
  bool fast = !s_over;
  int n_S = 0;
  int n_K = 0;                   // fast path: the kept members are list[0, n_K) after the decision

  if (fast) {
    // the row's min-p set: listed entries with z - zmax >= ln(min_p)
    auto push = [&](bool take, u64 e) {   // all lanes of the wave call it
      const u64 bm = __ballot(take);
      if (bm) {
        const int leader = __ffsll((long long)bm) - 1;
        unsigned int base = 0;
        if (lane == leader) base = atomicAdd(&s_n, (unsigned int)__popcll(bm));
        base = lane_value(base, leader);
        const unsigned int slot = base + (unsigned int)__popcll(bm & lanemask_lt());
        if (take && slot < (unsigned int)SCAP) list[slot] = e;
      }
    };
    auto member = [&](u64 e) { return key2f(sk_key(e)) - c.zmax >= c.ln_min_p; };
    {
      bool take[SPEC_R];
#pragma unroll
      for (int r = 0; r < SPEC_R; ++r) {
        const int idx = tid + r * PB, b = idx / per;
        take[r] = b < nb && (unsigned int)(idx - b * per) < s_cnt[min(b, nb - 1)] && member(spec[r]);
      }
      wave_append(take, &s_n, [&](int r, unsigned int slot) {
        if (slot < (unsigned int)SCAP) list[slot] = spec[r];
      });
    }
    for (int b = 0; b < nb; ++b) {   // lists longer than `per`
      const int cb = (int)s_cnt[b];
      for (int j0 = per; j0 < cb; j0 += PB) {
        const int j = j0 + tid;
        const u64 e = j < cb ? cand[(int64_t)b * CAP_B + j] : 0ull;
        push(j < cb && member(e), e);
      }
    }
    bar();
    n_S = (int)s_n;
    fast = n_S <= SCAP;
  }

  if (fast) {
    // mass of S and of its lightest member (one pair of barriers for both)
    u64 tot = 0, emin = ~0ull;
    for (int j = tid; j < n_S; j += PB) {
      const u64 ef = to_fix(__expf(key2f(sk_key(list[j])) - c.zmax));
      tot += ef;
      emin = ef < emin ? ef : emin;
    }
    tot = wave_reduce(tot, OpAdd());
    emin = wave_reduce(emin, OpMinU());
    if (lane == 0) {
      red64[wave] = tot;
      red64b[wave] = emin;
    }
    bar();
    tot = 0;
    emin = ~0ull;
    for (int w = 0; w < NW; ++w) {
      tot += red64[w];
      emin = red64b[w] < emin ? red64b[w] : emin;
    }
    bar();
    if (c.all_top || n_S == 0 || tot - emin <= P) {
      // the last member of S in order has mass tot - emin before it: all of S is kept
      c.all_top = true;
      W = tot;
      n_K = n_S;
    } else {
      const int n_pad = pow2_at_least(n_S);
      for (int j = n_S + tid; j < n_pad; j += PB) list[j] = ~0ull;
      if (tid == 0) {
        s_k = -1;
        s_first = INT_MAX;
        s_last = -1;
      }
      bar();
      bitonic_sort(list, n_pad);
      // exclusive prefix masses; thread t owns the run [t*R, (t+1)*R) of the sorted list
      const int R = (n_pad + PB - 1) / PB;
      const int j0 = tid * R;
      u64 run = 0;
      for (int r = 0; r < R; ++r) {
        const int j = j0 + r;
        if (j < n_S) run += to_fix(__expf(key2f(sk_key(list[j])) - c.zmax));
      }
      u64 total;
      u64 excl = block_scan(run, red64, &total);
      int k_loc = -1;
      u64 w_loc = 0;
      for (int r = 0; r < R; ++r) {
        const int j = j0 + r;
        if (j < n_S) {
          const u64 ef = to_fix(__expf(key2f(sk_key(list[j])) - c.zmax));
          if (excl <= P) {   // kept members form the prefix list[0, k]
            k_loc = j;
            w_loc = excl + ef;
          }
          excl += ef;
        }
      }
      if (k_loc >= 0) atomicMax(&s_k, k_loc);
      bar();
      const int k = s_k;   // >= 0: the first member has no mass before it
      if (k_loc == k) s_w = w_loc;
      const unsigned int ck = sk_key(list[k]);
      for (int j = tid; j < n_S; j += PB)
        if (sk_key(list[j]) == ck) {
          atomicMin(&s_first, j);
          atomicMax(&s_last, j);
        }
      bar();
      const int f = s_first, l = s_last;
      W = s_w;
      n_K = k + 1;
      c.cut = ck;
      c.ties_kept = (unsigned int)(k - f + 1);
      c.rank_ties = k < l;
      if (c.rank_ties) {   // the ties are sorted by id: count those below the chunk
        unsigned int t = 0;
        for (int j = f + tid; j <= l; j += PB) t += sk_id(list[j]) < i0;
        tie_before = block_sum(t, redu);
      }
    }
  } else {
    // ---- radix select over the whole row ----
    u64* hmass = list;
    for (int b = tid; b < H1; b += PB) {
      hmass[b] = 0ull;
      hcnt[b] = 0u;
    }
    bar();
    u64 smass = 0;   // mass of the min-p set
    const bool top = !c.all_top;
    strided_pass(z, 0, V, [&](int, float v) {
      const u64 ef = to_fix(__expf(v - c.zmax));
      if (v - c.zmax >= c.ln_min_p) smass += ef;
      if (top) {
        const unsigned int b = f2key(v) >> (32 - H1_BITS);
        atomicAdd(&hmass[b], ef);
        atomicAdd(&hcnt[b], 1u);
      }
    });
    smass = block_sum(smass, red64);   // its barriers also retire the LDS atomics
    if (!top) {
      W = smass;
    } else {
      u64 above;
      unsigned int prefix = (unsigned int)crossing_bin(hmass, hcnt, H1, P, red64, &s_low, &s_above, &above);
      u64 Pr = P - above;
      int shift = 32 - H1_BITS;
      unsigned int cut_count = 0;
      for (int pass = 0; pass < 2; ++pass) {
        const int new_shift = shift - 10;
        for (int b = tid; b < H2; b += PB) {
          hmass[b] = 0ull;
          hcnt[b] = 0u;
          hbefore[b] = 0u;
        }
        bar();
        strided_pass(z, 0, V, [&](int i, float v) {
          const unsigned int key = f2key(v);
          if ((key >> shift) == prefix) {
            const unsigned int b = (key >> new_shift) & (H2 - 1);
            atomicAdd(&hmass[b], to_fix(__expf(v - c.zmax)));
            atomicAdd(&hcnt[b], 1u);
            if (i < i0) atomicAdd(&hbefore[b], 1u);
          }
        });
        bar();
        const int b = crossing_bin(hmass, hcnt, H2, Pr, red64, &s_low, &s_above, &above);
        Pr -= above;
        if (pass == 1) {
          cut_count = hcnt[b];
          tie_before = hbefore[b];
        }
        prefix = (prefix << 10) | (unsigned int)b;
        shift = new_shift;
      }
      c.cut = prefix;
      // the t-th tie at the cut (0-based, ids ascending) has mass above + t * ecut before it
      const u64 ecut = to_fix(__expf(key2f(c.cut) - c.zmax));
      const u64 nt = ecut ? Pr / ecut + 1ull : (u64)cut_count;
      c.ties_kept = nt < cut_count ? (unsigned int)nt : cut_count;
      c.rank_ties = c.ties_kept < cut_count;
      // kept: the top-p prefix if its last key passes min-p, else the min-p set
      W = key2f(c.cut) - c.zmax >= c.ln_min_p ? (P - Pr) + (u64)c.ties_kept * ecut : smass;
    }
  }

  // ---- keep mask and probabilities of the chunk ----
  const float inv = (float)((double)FIX_SCALE / (double)W);
  constexpr u64 MASK41 = (1ull << 41) - 1ull;
  uint8_t* keep = p.keep ? p.keep + (int64_t)row * V : nullptr;
  float* probs = p.probs ? p.probs + (int64_t)row * V : nullptr;
  if (fast) {
    // the kept members list[0, n_K) as (id << 41) | mass (mass <= 2^40)
    for (int j = tid; j < n_K; j += PB) {
      const u64 e = list[j];
      list[j] = ((u64)(unsigned int)sk_id(e) << 41) | to_fix(__expf(key2f(sk_key(e)) - c.zmax));
    }
    bar();
  }
  // ---- token, when the kept set is listed: the smallest id whose inclusive kept mass exceeds u * W ----
  const u64 target = p.token ? (u64)((double)p.u[row] * (double)W) : 0ull;
  if (fast && p.token) {
    // kept mass below the chunk and inside it, and the last kept id; the one
    // workgroup whose chunk holds the crossing (or the last kept id, when
    // rounding leaves no mass above the target) searches its members
    u64 below = 0, inside = 0;
    int last = -1;
    for (int j = tid; j < n_K; j += PB) {
      const int id = (int)(list[j] >> 41);
      const u64 e = list[j] & MASK41;
      below += id < i0 ? e : 0ull;
      inside += id >= i0 && id < i1 ? e : 0ull;
      last = max(last, id);
    }
    below = wave_reduce(below, OpAdd());
    inside = wave_reduce(inside, OpAdd());
    last = wave_reduce(last, OpMaxI());
    if (lane == 0) {
      red64[wave] = below;
      red64b[wave] = inside;
      redu[wave] = (unsigned int)(last + 1);
    }
    bar();
    below = inside = 0;
    last = -1;
    for (int w = 0; w < NW; ++w) {
      below += red64[w];
      inside += red64b[w];
      last = max(last, (int)redu[w] - 1);
    }
    const bool cross = below <= target && target < below + inside;
    const bool at_end = target >= W && last >= i0 && last < i1;
    if (at_end && tid == 0) p.token[row] = last;
    if (cross) {   // workgroup-uniform
      if (tid == 0) {
        s_tok = INT_MAX;
        s_n = 0u;
      }
      bar();
      // the chunk's members, compacted (the whole list is searched if they do not fit)
      constexpr int SMALL = H1 / 2;
      u64* small = reinterpret_cast<u64*>(hcnt);
      for (int j = tid; j < n_K; j += PB) {
        const int id = (int)(list[j] >> 41);
        if (id >= i0 && id < i1) {
          const unsigned int slot = atomicAdd(&s_n, 1u);
          if (slot < (unsigned int)SMALL) small[slot] = list[j];
        }
      }
      bar();
      const bool fits = s_n <= (unsigned int)SMALL;
      const u64* src = fits ? small : list;
      const int nsrc = fits ? (int)s_n : n_K;
      // member t: kept mass before it = below + chunk members with smaller ids
      for (int j = tid; j < nsrc; j += PB) {
        const int id = (int)(src[j] >> 41);
        if (id < i0 || id >= i1) continue;
        u64 pre = below;
        for (int q0 = 0; q0 < nsrc; q0 += 8) {
          u64 e[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) e[q] = q0 + q < nsrc ? src[q0 + q] : ~0ull;
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const int idq = (int)(e[q] >> 41);
            pre += e[q] != ~0ull && idq >= i0 && idq < id ? e[q] & MASK41 : 0ull;
          }
        }
        if (pre <= target && pre + (src[j] & MASK41) > target) s_tok = id;   // exactly one member
      }
      bar();   // also: the count array is free again for the chunk bitmap
      if (tid == 0 && s_tok != INT_MAX) p.token[row] = s_tok;
    }
  }
  if ((keep || probs) && fast && i1 - i0 <= H1 * 32) {
    // mark the chunk's kept ids in an LDS bitmap (the count array is free) and
    // read z only at kept ids
    unsigned int* kbits = hcnt;
    const int nwords = (i1 - i0 + 31) / 32;
    for (int w = tid; w < nwords; w += PB) kbits[w] = 0u;
    bar();
    for (int j = tid; j < n_K; j += PB) {
      const int id = (int)(list[j] >> 41);
      if (id >= i0 && id < i1) atomicOr(&kbits[(id - i0) >> 5], 1u << ((id - i0) & 31));
    }
    bar();
    // 4 ids per store when the rows allow it (chunk bounds are then multiples of 4)
    const bool vec = (V & 3) == 0 && (reinterpret_cast<uintptr_t>(p.keep) & 3) == 0 &&
                     (reinterpret_cast<uintptr_t>(p.probs) & 15) == 0;
    if (vec) {
      for (int g = i0 + 4 * tid; g < i1; g += 4 * PB) {
        const unsigned int kb = (kbits[(g - i0) >> 5] >> ((g - i0) & 31)) & 0xfu;
        if (keep)
          *reinterpret_cast<unsigned int*>(keep + g) =
              (kb & 1u) | ((kb >> 1) & 1u) << 8 | ((kb >> 2) & 1u) << 16 | ((kb >> 3) & 1u) << 24;
        if (probs) {
          f32x4 pr = f32x4{0.f, 0.f, 0.f, 0.f};
          if (kb) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
              if ((kb >> q) & 1u) pr[q] = __expf(z[g + q] - c.zmax) * inv;
          }
          *reinterpret_cast<f32x4*>(probs + g) = pr;
        }
      }
    } else {
      for (int i = i0 + tid; i < i1; i += PB) {
        const bool k = (kbits[(i - i0) >> 5] >> ((i - i0) & 31)) & 1u;
        if (keep) keep[i] = (uint8_t)k;
        if (probs) probs[i] = k ? __expf(z[i] - c.zmax) * inv : 0.f;
      }
    }
  } else if (keep || probs) {
    unsigned int tie_run = tie_before;
    for (int s0 = i0; s0 < i1; s0 += SUBC) {
      float v[RPT];
      load_run(z, s0, i1, v);
      unsigned int tie_i = c.rank_ties ? wave_tie_base(v, s0, i1, c.cut, redu, tie_run) : 0u;
#pragma unroll
      for (int e = 0; e < RPT; ++e) {
        const int i = seg_id(s0, e);
        const bool valid = i < i1;
        const bool k = keep_step(c, v[e], valid, tie_i);
        if (valid && keep) keep[i] = (uint8_t)k;
        if (valid && probs) probs[i] = k ? __expf(v[e] - c.zmax) * inv : 0.f;
      }
    }
  }
  if (!p.token || fast) return;

  // radix-select path: the first workgroup scans the whole row, ids ascending
  if (blockIdx.x != 0) return;
  int last_kept;
  const int tok = ordered_token(z, 0, V, 0ull, target, c, red64, redu, &s_tok, &s_lastkept, &last_kept);
  if (tid == 0) p.token[row] = tok != INT_MAX ? tok : last_kept;
}

// ---- eta mode, passes 2 and 3 ----
// Row statistics from the chunk partials, computed by each calling wave (all
// lanes get them): row max, mass Z (chunk sums rescaled to the row max, fixed
// order) and the pool threshold ln(min(1, eta Z)). Both passes compute them
// from the same partials in the same order, so they agree bit for bit.
struct EtaStats {
  float zmax, lnthr;
};
__device__ inline EtaStats eta_row_stats(const PenaltyParams& p, const PenWs& ws, int row, int nb) {
  const int lane = threadIdx.x & 63;
  const float mb = lane < nb ? ws.pm[row * NBR_MAX + lane] : -INFINITY;
  const float sb = lane < nb ? ws.ps[row * NBR_MAX + lane] : 0.f;
  const float zb = lane < nb ? ws.pz[row * NBR_MAX + lane] : 0.f;
  const float zm = wave_reduce(mb, OpMax());
  const double sc = mb > -INFINITY ? (double)__expf(mb - zm) : 0.0;
  const double t = wave_reduce((double)sb * sc, OpAdd());
  const double ez = wave_reduce((double)zb * sc, OpAdd());
  const double H = log(t) + (double)zm - ez / t;   // nats
  const double eta = fmin((double)p.eta_eps, (double)p.eta_alpha * exp(-H));
  EtaStats r;
  r.zmax = zm;
  r.lnthr = (float)log(fmin(1.0, eta * t));   // -inf when eta = 0
  return r;
}

// z of the chunk: in registers (ZR per thread, -inf past i1) when it fits,
// the loads issued before the row statistics are formed. With `vec` (rows of
// a multiple of 4 ids, 16-byte aligned, so chunk bounds are multiples of 4)
// slot u holds id i0 + 4 (tid + (u / 4) PB) + u % 4 and four ids move per
// access; otherwise slot u holds id i0 + tid + u PB.
__device__ inline int chunk_slot(bool vec, int i0, int u) {
  const int tid = (int)threadIdx.x;
  return vec ? i0 + 4 * (tid + (u >> 2) * PB) + (u & 3) : i0 + tid + u * PB;
}
__device__ inline void load_chunk(const float* z, int i0, int i1, bool vec, float (&v)[ZR]) {
  if (vec) {
#pragma unroll
    for (int q = 0; q < ZR / 4; ++q) {
      const int g = chunk_slot(true, i0, 4 * q);
      const f32x4 t = g < i1 ? *reinterpret_cast<const f32x4*>(z + g) : f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
      for (int c = 0; c < 4; ++c) v[4 * q + c] = t[c];
    }
  } else {
#pragma unroll
    for (int u = 0; u < ZR; ++u) {
      const int i = chunk_slot(false, i0, u);
      v[u] = i < i1 ? z[i] : -INFINITY;
    }
  }
}

// Pass 2: the chunk's kept mass (fixed point) and last kept id.
__global__ __launch_bounds__(PB) void pen_eta_mass_kernel(const PenaltyParams p, int nb) {
  __shared__ u64 red64[NW];
  __shared__ int redi[NW];
  const int row = blockIdx.y, tid = threadIdx.x;
  const PenWs ws = carve(p.ws, p.rows);
  int i0, i1;
  chunk_of(p.V, nb, blockIdx.x, &i0, &i1);
  const float* z = p.logits_out + (int64_t)row * p.V;
  const bool in_regs = i1 - i0 <= ZR * PB;
  const bool vec = (p.V & 3) == 0 && (reinterpret_cast<uintptr_t>(p.logits_out) & 15) == 0;
  float v[ZR];
  if (in_regs) load_chunk(z, i0, i1, vec, v);
  const EtaStats st = eta_row_stats(p, ws, row, nb);
  u64 m = 0;
  int last = -1;
  auto take = [&](int i, float w) {
    if (w - st.zmax >= st.lnthr) {   // the keep test of the other passes
      m += to_fix(__expf(w - st.zmax));
      last = i;
    }
  };
  if (in_regs) {
#pragma unroll
    for (int u = 0; u < ZR; ++u) {
      const int i = chunk_slot(vec, i0, u);
      if (i < i1) take(i, v[u]);
    }
  } else {
    strided_pass(z, i0, i1, take);
  }
  m = block_sum(m, red64);
  last = wave_reduce(last, OpMaxI());
  if ((tid & 63) == 0) redi[tid >> 6] = last;
  bar();
  if (tid == 0) {
    for (int w = 0; w < NW; ++w) last = max(last, redi[w]);
    ws.pw[row * NBR_MAX + blockIdx.x] = m;
    ws.pl[row * NBR_MAX + blockIdx.x] = last;
  }
}

// Pass 3: keep mask, probabilities and token of the chunk.
__global__ __launch_bounds__(PB) void pen_eta_out_kernel(const PenaltyParams p, int nb) {
  __shared__ u64 red64[NW];
  __shared__ unsigned int redu[NW];
  __shared__ int s_tok, s_lastkept;
  const int row = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
  const PenWs ws = carve(p.ws, p.rows);
  const int V = p.V;
  int i0, i1;
  chunk_of(V, nb, blockIdx.x, &i0, &i1);
  const float* z = p.logits_out + (int64_t)row * V;
  const bool in_regs = i1 - i0 <= ZR * PB;
  // four ids per access when the rows and the outputs allow it
  const bool vec = (V & 3) == 0 && (reinterpret_cast<uintptr_t>(p.logits_out) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(p.keep) & 3) == 0 && (reinterpret_cast<uintptr_t>(p.probs) & 15) == 0;
  float v[ZR];
  if (in_regs && (p.keep || p.probs)) load_chunk(z, i0, i1, vec, v);
  const EtaStats st = eta_row_stats(p, ws, row, nb);
  // kept mass of the row and below the chunk, the row's last kept id (every wave)
  const u64 wb = lane < nb ? ws.pw[row * NBR_MAX + lane] : 0ull;
  const int lb = lane < nb ? ws.pl[row * NBR_MAX + lane] : -1;
  const u64 W = wave_reduce(wb, OpAdd());
  const u64 below = wave_reduce(lane < (int)blockIdx.x ? wb : 0ull, OpAdd());
  const u64 inside = lane_value(wb, (int)blockIdx.x);
  const int last = wave_reduce(lb, OpMaxI());
  Cut c;
  c.zmax = st.zmax;
  c.ln_min_p = st.lnthr;
  c.all_top = true;
  c.rank_ties = false;
  c.cut = 0u;
  c.ties_kept = 0u;
  const float inv = (float)((double)FIX_SCALE / (double)W);
  uint8_t* keep = p.keep ? p.keep + (int64_t)row * V : nullptr;
  float* probs = p.probs ? p.probs + (int64_t)row * V : nullptr;
  auto put = [&](int i, float w) {
    const bool k = w - c.zmax >= c.ln_min_p;
    if (keep) keep[i] = (uint8_t)k;
    if (probs) probs[i] = k ? __expf(w - c.zmax) * inv : 0.f;
  };
  if (keep || probs) {
    if (in_regs && vec) {
#pragma unroll
      for (int q = 0; q < ZR / 4; ++q) {
        const int g = chunk_slot(true, i0, 4 * q);
        if (g < i1) {
          unsigned int kb = 0;
          f32x4 pr;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float w = v[4 * q + e];
            const bool k = w - c.zmax >= c.ln_min_p;
            kb |= (k ? 1u : 0u) << (8 * e);
            pr[e] = k ? __expf(w - c.zmax) * inv : 0.f;
          }
          if (keep) *reinterpret_cast<unsigned int*>(keep + g) = kb;
          if (probs) *reinterpret_cast<f32x4*>(probs + g) = pr;
        }
      }
    } else if (in_regs) {
#pragma unroll
      for (int u = 0; u < ZR; ++u) {
        const int i = chunk_slot(false, i0, u);
        if (i < i1) put(i, v[u]);
      }
    } else {
      strided_pass(z, i0, i1, put);
    }
  }
  if (!p.token) return;
  // the smallest id whose inclusive kept mass exceeds u W; the last kept id
  // when rounding leaves no mass above the target
  const u64 target = (u64)((double)p.u[row] * (double)W);
  if (target >= W) {   // the chunk holding the last kept id writes it (-1 from the first chunk if none)
    if (tid == 0 && ((last >= i0 && last < i1) || (last < 0 && blockIdx.x == 0))) p.token[row] = last;
  } else if (below <= target && target < below + inside) {   // workgroup-uniform
    int lk;
    const int tok = ordered_token(z, i0, i1, below, target, c, red64, redu, &s_tok, &s_lastkept, &lk);
    if (tid == 0) p.token[row] = tok != INT_MAX ? tok : lk;
  }
}

}  // namespace

size_t penalty_workspace_bytes(int32_t rows, int32_t V) { return pen_ws_bytes(rows, V); }

hipError_t launch_penalty(const PenaltyParams& p, hipStream_t stream) {
  const int nb = penalty_blocks_per_row(p.rows, p.V);
  const dim3 grid(nb, p.rows);
  hipLaunchKernelGGL(pen_z_kernel, grid, dim3(PB), 0, stream, p, nb);
  if (!(p.keep || p.probs || p.token)) return hipGetLastError();
  if (p.eta_mode) {
    hipLaunchKernelGGL(pen_eta_mass_kernel, grid, dim3(PB), 0, stream, p, nb);
    hipLaunchKernelGGL(pen_eta_out_kernel, grid, dim3(PB), 0, stream, p, nb);
  } else {
    hipLaunchKernelGGL(pen_out_kernel, grid, dim3(PB), 0, stream, p, nb);
  }
  return hipGetLastError();
}

}  // namespace ts
