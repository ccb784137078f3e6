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

struct Smem {
  unsigned int bitmap[MAX_V / 32];
  unsigned long long hmass[H1];
  unsigned int hcnt[H1];
  unsigned long long red64[NWAVES];
  float redf[NWAVES];
  unsigned int redu[NWAVES];
  int bin;
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

__device__ inline float block_sum(float x, Smem& s) {
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  if ((threadIdx.x & 63) == 0) s.redf[threadIdx.x >> 6] = x;
  __syncthreads();
  float r = 0.f;
  for (int w = 0; w < NWAVES; ++w) r += s.redf[w];
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

__device__ inline unsigned int block_scan32(unsigned int x, Smem& s, unsigned int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  unsigned int incl = x;
  for (int off = 1; off < 64; off <<= 1) {
    const unsigned int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) s.redu[wave] = incl;
  __syncthreads();
  unsigned int pre = 0, tot = 0;
  for (int w = 0; w < NWAVES; ++w) {
    if (w < wave) pre += s.redu[w];
    tot += s.redu[w];
  }
  __syncthreads();
  *total = tot;
  return pre + incl - x;
}

__device__ inline float block_scanf(float x, Smem& s, float* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float incl = x;
  for (int off = 1; off < 64; off <<= 1) {
    const float y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) s.redf[wave] = incl;
  __syncthreads();
  float pre = 0.f, tot = 0.f;
  for (int w = 0; w < NWAVES; ++w) {
    if (w < wave) pre += s.redf[w];
    tot += s.redf[w];
  }
  __syncthreads();
  *total = tot;
  return pre + (incl - x);
}

__global__ __launch_bounds__(PT_THREADS) void penalty_kernel(const PenaltyParams p) {
  __shared__ Smem s;
  __shared__ int s_lowbin;
  __shared__ unsigned long long s_above;
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int V = p.V;
  const float* x = p.logits + (int64_t)row * V;
  float* z = p.logits_out + (int64_t)row * V;

  // 0. window bitmap
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

  // 1. penalty, temperature, max
  float mx = -INFINITY;
  for (int i = tid; i < V; i += PT_THREADS) {
    float v = x[i];
    if ((s.bitmap[i >> 5] >> (i & 31)) & 1u) v = v > 0.f ? v / p.penalty : v * p.penalty;
    v = v / p.temperature;
    z[i] = v;
    mx = fmaxf(mx, v);
  }
  const float zmax = block_max(mx, s);
  const float ln_min_p = logf(p.min_p);  // -inf for min_p = 0

  // 2. mass histogram over the top 12 key bits, total mass (fixed point)
  const bool all_top = p.top_p >= 1.0f;
  unsigned int cut = 0u;          // keys above `cut` are kept by top-p
  unsigned int cut_ties = 0u;     // ties at `cut` kept, earliest ids first
  unsigned int cut_count = 0u;    // ties at `cut` in the row
  if (!all_top) {
    for (int b = tid; b < H1; b += PT_THREADS) {
      s.hmass[b] = 0ull;
      s.hcnt[b] = 0u;
    }
    __syncthreads();
    unsigned long long zsum = 0;
    for (int i = tid; i < V; i += PT_THREADS) {
      const float v = z[i];
      const unsigned long long f = to_fix(__expf(v - zmax));
      const unsigned int b = f2key(v) >> (32 - H1_BITS);
      atomicAdd(&s.hmass[b], f);
      atomicAdd(&s.hcnt[b], 1u);
      zsum += f;
    }
    const unsigned long long Z = block_sum64(zsum, s);
    unsigned long long P = (unsigned long long)((double)p.top_p * (double)Z);

    // crossing search: digit 1 (12 bits), then 2 x 10 bits
    unsigned int prefix = 0u;
    int shift = 32;
    for (int pass = 0; pass < 3; ++pass) {
      const int nbits = pass == 0 ? H1_BITS : 10;
      const int nb = 1 << nbits;
      const int new_shift = shift - nbits;
      if (pass > 0) {
        __syncthreads();
        for (int b = tid; b < nb; b += PT_THREADS) {
          s.hmass[b] = 0ull;
          s.hcnt[b] = 0u;
        }
        __syncthreads();
        for (int i = tid; i < V; i += PT_THREADS) {
          const float v = z[i];
          const unsigned int key = f2key(v);
          if ((key >> shift) == prefix) {
            const unsigned int b = (key >> new_shift) & (nb - 1);
            atomicAdd(&s.hmass[b], to_fix(__expf(v - zmax)));
            atomicAdd(&s.hcnt[b], 1u);
          }
        }
        __syncthreads();
      }
      // lowest non-empty bin whose exclusive mass from the top is <= P
      const int per = nb / PT_THREADS > 0 ? nb / PT_THREADS : 1;
      const bool owner = tid * per < nb;
      const int hi_bin = nb - 1 - tid * per;
      unsigned long long m = 0;
      if (owner)
        for (int i = 0; i < per; ++i) m += s.hmass[hi_bin - i];
      if (tid == 0) s_lowbin = nb;
      unsigned long long tot;
      const unsigned long long before = block_scan64(m, s, &tot);
      if (owner) {
        unsigned long long acc = before;
        int best = nb;
        for (int i = 0; i < per; ++i) {
          const int b = hi_bin - i;
          if (s.hcnt[b] && acc <= P) best = b;
          acc += s.hmass[b];
        }
        if (best < nb) atomicMin(&s_lowbin, best);
      }
      __syncthreads();
      const int b = s_lowbin;
      // exclusive mass above bin b (recomputed by the owner of b)
      if (owner && b <= hi_bin && b > hi_bin - per) {
        unsigned long long acc = before;
        for (int i = 0; i < per; ++i) {
          if (hi_bin - i == b) break;
          acc += s.hmass[hi_bin - i];
        }
        s_above = acc;
      }
      __syncthreads();
      P -= s_above;
      if (pass == 2) cut_count = s.hcnt[b];
      prefix = (prefix << nbits) | (unsigned int)b;
      shift = new_shift;
    }
    cut = prefix;
    const unsigned long long ecut = to_fix(__expf(key2f(cut) - zmax));
    // ties at the cut: the t-th (0-based, ids ascending) has mass-before = A + t * ecut
    unsigned long long nt = ecut ? P / ecut + 1ull : (unsigned long long)cut_count;
    cut_ties = nt < cut_count ? (unsigned int)nt : cut_count;
    __syncthreads();
  }

  // 5./6. keep mask, kept mass, then probabilities and token. Elements are
  // visited in rounds of 4 consecutive ids per thread so that ties at the cut
  // are ranked by id with a block scan (only needed when some ties drop out).
  const bool rank_ties = !all_top && cut_ties < cut_count;
  auto round_keep = [&](int base, float* ev, unsigned int* kept_bits, unsigned int* tie_run) {
    unsigned int tflags = 0u, gflags = 0u;
    float zv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = base + 4 * tid + e;
      zv[e] = -INFINITY;
      if (i < V) {
        zv[e] = z[i];
        const unsigned int key = f2key(zv[e]);
        gflags |= (unsigned int)(all_top || key > cut) << e;
        tflags |= (unsigned int)(!all_top && key == cut) << e;
      }
    }
    unsigned int tie_b = 0u;
    if (rank_ties) {
      unsigned int total;
      tie_b = *tie_run + block_scan32(__popc(tflags), s, &total);
      *tie_run += total;
    }
    unsigned int kb = 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = base + 4 * tid + e;
      bool top = (gflags >> e) & 1u;
      if ((tflags >> e) & 1u) {
        top = !rank_ties || tie_b < cut_ties;
        ++tie_b;
      }
      const float d = zv[e] - zmax;
      const bool k = i < V && top && d >= ln_min_p;
      ev[e] = k ? __expf(d) : 0.f;
      kb |= (unsigned int)k << e;
    }
    *kept_bits = kb;
  };

  float kept_sum = 0.f;
  {
    unsigned int tie_run = 0u;
    for (int base = 0; base < V; base += 4 * PT_THREADS) {
      float ev[4];
      unsigned int kb;
      round_keep(base, ev, &kb, &tie_run);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = base + 4 * tid + e;
        if (i < V && p.keep) p.keep[(int64_t)row * V + i] = (uint8_t)((kb >> e) & 1u);
        kept_sum += ev[e];
      }
    }
  }
  const float S = block_sum(kept_sum, s);
  if (!p.probs && !p.token) return;

  const float target = p.u ? p.u[row] * S : 0.f;
  float run = 0.f;
  int found = -1;
  int last_kept = -1;
  unsigned int tie_run = 0u;
  __shared__ int s_tok;
  if (tid == 0) s_tok = 0x7fffffff;
  for (int base = 0; base < V; base += 4 * PT_THREADS) {
    float ev[4];
    unsigned int kb;
    round_keep(base, ev, &kb, &tie_run);
    const float inv = 1.0f / S;
    float local = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = base + 4 * tid + e;
      if (i < V && p.probs) p.probs[(int64_t)row * V + i] = ev[e] * inv;
      local += ev[e];
      if ((kb >> e) & 1u) last_kept = i;
    }
    if (p.token && found < 0) {
      float total;
      const float before = run + block_scanf(local, s, &total);
      float acc = before;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc += ev[e];
        if (((kb >> e) & 1u) && acc > target && before <= target) {
          // first element of this thread to cross; threads are in id order
          atomicMin(&s_tok, base + 4 * tid + e);
          break;
        }
      }
      __syncthreads();
      if (s_tok != 0x7fffffff) found = s_tok;
      run += total;
      __syncthreads();
    }
  }
  if (p.token) {
    // rounding may leave u*S just above the last cumulative sum: take the last kept id
    __shared__ int s_last;
    if (tid == 0) s_last = -1;
    __syncthreads();
    atomicMax(&s_last, last_kept);
    __syncthreads();
    if (tid == 0) p.token[row] = found >= 0 ? found : s_last;
  }
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
