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
// One 1024-thread workgroup per row, passes over the row (L2-resident after
// the first):
//   0. window ids -> LDS bitmap (set semantics makes duplicates harmless);
//   1. penalty + temperature -> logits_out, row max;
//   2. e_i = exp(z_i - max) as 2^-40 fixed point; histogram of mass and count
//      over the top 12 bits of the order-preserving key of z (integer LDS
//      atomics, so the sums do not depend on thread timing); total mass;
//   3-4. two 10-bit radix refinements inside the bin where the mass from the
//      top crosses top_p * total -> the exact cut key, the mass above it and
//      how many of its ties (ids ascending) stay;
//   5. keep mask (top-p and min-p), kept mass;
//   6. renormalised probabilities and the inverse-CDF token (ordered scan).
// Passes 3-4 are skipped when top_p >= 1, pass 6 when neither probs nor a
// token is requested.
#include "ts_internal.h"

#include <cmath>

namespace ts {
namespace {

constexpr int PT_THREADS = 1024;
constexpr int NWAVES = PT_THREADS / 64;
constexpr int H1_BITS = 12;
constexpr int H1 = 1 << H1_BITS;
constexpr int MAX_V = 262144;
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

constexpr int NCAND = MAX_V / 32;  // candidate keys of the cut bin, in the bitmap's space

struct Smem {
  union {
    unsigned int bitmap[MAX_V / 32];   // window ids (passes 0-1)
    unsigned int cand[NCAND];          // keys of the top-p cut bin (after pass 1)
  };
  unsigned long long hmass[H1];
  unsigned int hcnt[H1];
  unsigned long long red64[NWAVES];
  float redf[NWAVES];
  unsigned int redu[NWAVES];
  float wmass[NWAVES];                 // kept mass of each wave's id segment
  unsigned int wtie[NWAVES];           // ties at the cut in each wave's segment
  int lowbin;
  unsigned long long above;
  unsigned int ncand;
  int tok;
  int last;
};

__device__ inline float block_max(float x, Smem& s) {
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
  if ((threadIdx.x & 63) == 0) s.redf[threadIdx.x >> 6] = x;
  __syncthreads();
  float r = s.redf[0];
  for (int w = 1; w < NWAVES; ++w) r = fmaxf(r, s.redf[w]);
  __syncthreads();
  return r;
}

__device__ inline unsigned long long block_sum64(unsigned long long x, Smem& s) {
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  if ((threadIdx.x & 63) == 0) s.red64[threadIdx.x >> 6] = x;
  __syncthreads();
  unsigned long long r = 0;
  for (int w = 0; w < NWAVES; ++w) r += s.red64[w];
  __syncthreads();
  return r;
}

// Exclusive prefix over threads (thread order) of a 64-bit value; *total gets the sum.
__device__ inline unsigned long long block_scan64(unsigned long long x, Smem& s, unsigned long long* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  unsigned long long incl = x;
  for (int off = 1; off < 64; off <<= 1) {
    const unsigned long long y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) s.red64[wave] = incl;
  __syncthreads();
  unsigned long long pre = 0, tot = 0;
  for (int w = 0; w < NWAVES; ++w) {
    if (w < wave) pre += s.red64[w];
    tot += s.red64[w];
  }
  __syncthreads();
  *total = tot;
  return pre + incl - x;
}

__device__ inline unsigned long long lanemask_lt() { return (1ull << (threadIdx.x & 63)) - 1ull; }

// Lowest non-empty bin of s.hmass/s.hcnt[0, nb) whose mass from the top
// (exclusive) is <= P; returns it and its exclusive mass above.
__device__ inline int crossing_bin(int nb, unsigned long long P, Smem& s, unsigned long long* above) {
  const int tid = threadIdx.x;
  const int per = nb / PT_THREADS > 0 ? nb / PT_THREADS : 1;
  const bool owner = tid * per < nb;
  const int hi_bin = nb - 1 - tid * per;
  unsigned long long m = 0;
  if (owner)
    for (int i = 0; i < per; ++i) m += s.hmass[hi_bin - i];
  if (tid == 0) s.lowbin = nb;
  unsigned long long tot;
  const unsigned long long before = block_scan64(m, s, &tot);  // ends with a barrier
  if (owner) {
    unsigned long long acc = before;
    int best = nb;
    for (int i = 0; i < per; ++i) {
      const int b = hi_bin - i;
      if (s.hcnt[b] && acc <= P) best = b;
      acc += s.hmass[b];
    }
    if (best < nb) atomicMin(&s.lowbin, best);
  }
  __syncthreads();
  const int b = s.lowbin;
  if (owner && b <= hi_bin && b > hi_bin - per) {
    unsigned long long acc = before;
    for (int i = 0; i < per && hi_bin - i != b; ++i) acc += s.hmass[hi_bin - i];
    s.above = acc;
  }
  __syncthreads();
  *above = s.above;
  return b;
}

constexpr int UNR = 32;  // loads in flight per thread in every pass (~128 KB per CU)

// Thread-strided pass over n floats with UNR loads issued before any use.
template <typename F>
__device__ inline void strided_pass(const float* src, int n, F&& f) {
  for (int i0 = threadIdx.x; i0 < n; i0 += UNR * PT_THREADS) {
    float v[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int i = i0 + u * PT_THREADS;
      v[u] = i < n ? src[i] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int i = i0 + u * PT_THREADS;
      if (i < n) f(i, v[u]);
    }
  }
}

// Ordered pass of one wave over ids [s0, s1), 64 ids per step in ascending
// order, UNR steps' loads in flight. f(i, valid, value) is called by all lanes
// (it may use ballots); wave-uniform bounds.
template <typename F>
__device__ inline void wave_pass(const float* src, int s0, int s1, F&& f) {
  const int lane = threadIdx.x & 63;
  for (int b0 = s0; b0 < s1; b0 += UNR * 64) {
    float v[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int i = b0 + u * 64 + lane;
      v[u] = i < s1 ? src[i] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int i = b0 + u * 64 + lane;
      if (b0 + u * 64 < s1) f(i, i < s1, v[u]);
    }
  }
}

// Append `key` to s.cand when `take`: one LDS atomic per wave (ballot + rank).
__device__ inline void append_cand(bool take, unsigned int key, Smem& s) {
  const unsigned long long m = __ballot(take);
  if (!m) return;
  const int leader = __ffsll((long long)m) - 1;
  unsigned int base = 0;
  if ((int)(threadIdx.x & 63) == leader) base = atomicAdd(&s.ncand, (unsigned int)__popcll(m));
  base = __shfl(base, leader);
  if (take) s.cand[base + (unsigned int)__popcll(m & lanemask_lt())] = key;
}

__global__ __launch_bounds__(PT_THREADS) void penalty_kernel(const PenaltyParams p) {
  __shared__ Smem s;
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int V = p.V;
  const float* x = p.logits + (int64_t)row * V;
  float* z = p.logits_out + (int64_t)row * V;

  // 0. window bitmap (set semantics: duplicates are harmless)
  const int nwords = (V + 31) / 32;
  for (int w = tid; w < nwords; w += PT_THREADS) s.bitmap[w] = 0u;
  __syncthreads();
  if (p.W > 0) {
    const int32_t* win = p.window + (int64_t)row * p.window_stride;
    for (int w = tid; w < p.W; w += PT_THREADS) {
      const int id = win[w];
      if (id >= 0 && id < V) atomicOr(&s.bitmap[id >> 5], 1u << (id & 31));
    }
  }
  __syncthreads();

  // 1. penalty, temperature, row max
  float mx = -INFINITY;
  strided_pass(x, V, [&](int i, float v) {
    if ((s.bitmap[i >> 5] >> (i & 31)) & 1u) v = v > 0.f ? v / p.penalty : v * p.penalty;
    v = v / p.temperature;
    z[i] = v;
    mx = fmaxf(mx, v);
  });
  const float zmax = block_max(mx, s);  // its barriers also retire the bitmap
  const float ln_min_p = logf(p.min_p);  // -inf for min_p = 0

  // 2. top-p cut: mass histogram over the top 12 key bits (2^-40 fixed point,
  // integer LDS atomics), then two 10-bit refinements inside the bin where the
  // mass counted from the top crosses top_p * total.
  const bool all_top = p.top_p >= 1.0f;
  unsigned int cut = 0u, cut_ties = 0u, cut_count = 0u;
  if (!all_top) {
    for (int b = tid; b < H1; b += PT_THREADS) {
      s.hmass[b] = 0ull;
      s.hcnt[b] = 0u;
    }
    if (tid == 0) s.ncand = 0;
    __syncthreads();
    unsigned long long zsum = 0;
    strided_pass(z, V, [&](int, float v) {
      const unsigned long long f = to_fix(__expf(v - zmax));
      const unsigned int b = f2key(v) >> (32 - H1_BITS);
      atomicAdd(&s.hmass[b], f);
      atomicAdd(&s.hcnt[b], 1u);
      zsum += f;
    });
    const unsigned long long Z = block_sum64(zsum, s);
    unsigned long long P = (unsigned long long)((double)p.top_p * (double)Z);
    unsigned long long above;
    unsigned int prefix = (unsigned int)crossing_bin(H1, P, s, &above);
    P -= above;
    int shift = 32 - H1_BITS;
    const bool in_lds = s.hcnt[prefix] <= (unsigned int)NCAND;
    if (in_lds) {
      // every wave walks whole 64-id steps so the ballots see all lanes
      const int seg = ((V + NWAVES - 1) / NWAVES + 63) / 64 * 64;
      wave_pass(z, wave * seg, min(wave * seg + seg, V), [&](int, bool valid, float v) {
        const unsigned int key = f2key(v);
        append_cand(valid && (key >> shift) == prefix, key, s);
      });
    }
    for (int pass = 0; pass < 2; ++pass) {
      const int nb = 1 << 10;
      const int new_shift = shift - 10;
      __syncthreads();
      for (int b = tid; b < nb; b += PT_THREADS) {
        s.hmass[b] = 0ull;
        s.hcnt[b] = 0u;
      }
      __syncthreads();
      if (in_lds) {
        const unsigned int n = s.ncand;
        for (unsigned int i = tid; i < n; i += PT_THREADS) {
          const unsigned int key = s.cand[i];
          if ((key >> shift) == prefix) {
            const unsigned int b = (key >> new_shift) & (nb - 1);
            atomicAdd(&s.hmass[b], to_fix(__expf(key2f(key) - zmax)));
            atomicAdd(&s.hcnt[b], 1u);
          }
        }
      } else {
        strided_pass(z, V, [&](int, float v) {
          const unsigned int key = f2key(v);
          if ((key >> shift) == prefix) {
            const unsigned int b = (key >> new_shift) & (nb - 1);
            atomicAdd(&s.hmass[b], to_fix(__expf(v - zmax)));
            atomicAdd(&s.hcnt[b], 1u);
          }
        });
      }
      __syncthreads();
      const int b = crossing_bin(nb, P, s, &above);
      P -= above;
      if (pass == 1) cut_count = s.hcnt[b];
      prefix = (prefix << 10) | (unsigned int)b;
      shift = new_shift;
    }
    cut = prefix;
    const unsigned long long ecut = to_fix(__expf(key2f(cut) - zmax));
    // ties at the cut: the t-th (0-based, ids ascending) has mass before it = above + t * ecut
    const unsigned long long nt = ecut ? P / ecut + 1ull : (unsigned long long)cut_count;
    cut_ties = nt < cut_count ? (unsigned int)nt : cut_count;
  }

  // 3./4. keep mask, kept mass, probabilities and the token. Each wave owns a
  // contiguous id segment and walks it in order, so ties at the cut are ranked
  // by id with ballots, and the inverse CDF needs a single search.
  const bool rank_ties = !all_top && cut_ties < cut_count;
  const int seg = ((V + NWAVES - 1) / NWAVES + 63) / 64 * 64;
  const int s0 = min(wave * seg, V);
  const int s1 = min(s0 + seg, V);
  unsigned int tie_base = 0;
  if (rank_ties) {
    unsigned int c = 0;
    wave_pass(z, s0, s1, [&](int, bool valid, float v) { c += valid && f2key(v) == cut; });
    for (int m = 32; m >= 1; m >>= 1) c += __shfl_xor(c, m);
    if (lane == 0) s.wtie[wave] = c;
    __syncthreads();
    for (int w = 0; w < wave; ++w) tie_base += s.wtie[w];
  }
  // keep decision of an id (all lanes call it; tie_run counts ties of earlier ids)
  auto keep_of = [&](bool valid, float zv, unsigned int& tie_run) -> bool {
    const unsigned int key = f2key(zv);
    bool top = all_top || key > cut;
    const bool tie = valid && !all_top && key == cut;
    const unsigned long long tm = __ballot(tie);
    if (tie) top = !rank_ties || (tie_run + (unsigned int)__popcll(tm & lanemask_lt())) < cut_ties;
    tie_run += (unsigned int)__popcll(tm);
    return valid && top && (zv - zmax >= ln_min_p);
  };

  float wsum = 0.f;
  {
    unsigned int tie_run = tie_base;
    wave_pass(z, s0, s1, [&](int i, bool valid, float zv) {
      const bool k = keep_of(valid, zv, tie_run);
      if (valid && p.keep) p.keep[(int64_t)row * V + i] = (uint8_t)k;
      wsum += k ? __expf(zv - zmax) : 0.f;
    });
  }
  for (int m = 32; m >= 1; m >>= 1) wsum += __shfl_xor(wsum, m);
  if (lane == 0) s.wmass[wave] = wsum;
  if (tid == 0) {
    s.tok = -1;
    s.last = -1;
  }
  __syncthreads();
  float S = 0.f, wbase = 0.f;
  for (int w = 0; w < NWAVES; ++w) {
    if (w < wave) wbase += s.wmass[w];
    S += s.wmass[w];
  }
  if (!p.probs && !p.token) return;

  const float inv = 1.0f / S;
  const float target = p.u ? p.u[row] * S : 0.f;
  const bool mine = p.token && target >= wbase && target < wbase + s.wmass[wave];
  {
    unsigned int tie_run = tie_base;
    float run = wbase;
    bool done = false;
    int last_kept = -1;
    wave_pass(z, s0, s1, [&](int i, bool valid, float zv) {
      const bool k = keep_of(valid, zv, tie_run);
      const float e = k ? __expf(zv - zmax) : 0.f;
      if (valid && p.probs) p.probs[(int64_t)row * V + i] = e * inv;
      const unsigned long long km = __ballot(k);
      const int b0 = i - lane;
      if (km) last_kept = b0 + 63 - __clzll(km);
      if (mine && !done) {
        // inclusive prefix of e over the 64 lanes (ids ascending)
        float incl = e;
        for (int off = 1; off < 64; off <<= 1) {
          const float y = __shfl_up(incl, off);
          if (lane >= off) incl += y;
        }
        const unsigned long long hit = __ballot(k && run + incl > target);
        if (hit) {
          if (lane == 0) s.tok = b0 + __ffsll((long long)hit) - 1;
          done = true;
        }
        run += __shfl(incl, 63);
      }
    });
    if (lane == 0 && last_kept >= 0) atomicMax(&s.last, last_kept);
    if (mine && !done && lane == 0) s.tok = last_kept;  // rounding left u*S past this wave's sum
  }
  __syncthreads();
  // u*S may round to (or past) the total: fall back to the last kept id
  if (p.token && tid == 0) p.token[row] = s.tok >= 0 ? s.tok : s.last;
}

}  // namespace

size_t penalty_workspace_bytes(int32_t rows, int32_t V) {
  (void)rows;
  (void)V;
  return 0;
}

hipError_t launch_penalty(const PenaltyParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(penalty_kernel, dim3(p.rows), dim3(PT_THREADS), 0, stream, p);
  return hipGetLastError();
}

}  // namespace ts
