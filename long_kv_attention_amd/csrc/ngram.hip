// Token reutilisation for CDNA4 (gfx950): 4-gram retrieval over the recent
// window, random choice among the valid n-grams and the draft tree.
//
// What is computed (TokenSwift summary §3.2 "Multi-token Generation and
// Token Reutilization": frequent 4-grams of the generated text are reused as
// draft candidates, at most k retrieved; §3.4: a random choice among several
// valid n-grams; §4.4.1 and Appendix B.2: a ternary [1,3,3,3] tree):
//   * valid 4-grams are those of the window whose first token is the root
//     (the window's last token); they are counted per distinct continuation
//     and numbered in order of first occurrence;
//   * more than k distinct continuations: the k with the smallest
//     (SplitMix64 output q of the caller's seed, q) are kept (a uniformly
//     random subset);
//   * kept chains are ordered by count (descending), then first occurrence;
//   * tree: root, the head part (three candidates per level, each level
//     under the first node of the previous one), then the chains under the
//     root, cut at T_max nodes.
//
// One workgroup of 1024 threads does everything in LDS: the window, the
// continuations of the root's occurrences (a block scan keeps them in window
// order), per occurrence its continuation's count and distinct index
// (pairwise comparisons: the occurrences of one token are few in practice, at
// most W), the random keys of the distinct continuations, the choice and the
// order (ranks by counting), then one thread per tree node. The comparison
// loops read independent LDS words eight at a time, so their latencies
// overlap.
#include "ts_device.h"
#include "ts_internal.h"

namespace ts {
namespace {

constexpr int NG_T = 1024;                  // threads
constexpr int NG_SEG = NG_MAX_WINDOW / NG_T;  // window positions per thread in the scans
constexpr int NG_MAX_NODES = 128;                     // largest tree
constexpr int NG_MAX_CHAINS = (NG_MAX_NODES - 1) / 3 + 1;   // chains that can start inside a tree

__device__ inline u64 splitmix64(u64 seed, u64 j) {
  u64 z = seed + (j + 1ull) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Exclusive prefix sum over the 1024 threads' values (thread order); `tmp`
// holds one slot per wave. Every thread gets the total.
__device__ inline int block_scan(int x, int* tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = wave_incl_scan(x);
  if (lane == 63) tmp[wave] = incl;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NG_T / 64; ++w) {
    const int t = tmp[w];
    before += w < wave ? t : 0;
    tot += t;
  }
  __syncthreads();   // tmp is reused by the next scan
  *total = tot;
  return before + incl - x;
}

__global__ __launch_bounds__(NG_T) void ngram_tree_kernel(const NgramParams p) {
  __shared__ int32_t w[NG_MAX_WINDOW];     // the window
  __shared__ int32_t ka[NG_MAX_WINDOW];    // continuation (a, b, c) of the root's valid occurrences,
  __shared__ int32_t kb[NG_MAX_WINDOW];    // in window order
  __shared__ int32_t kc[NG_MAX_WINDOW];
  __shared__ int32_t cnt[NG_MAX_WINDOW];   // per occurrence: its continuation's count if first occurrence, else 0
  __shared__ int32_t dq[NG_MAX_WINDOW];    // per occurrence: distinct index if first occurrence, else -1
  __shared__ u64 rho[NG_MAX_WINDOW];       // per distinct index: random key
  __shared__ int32_t chain_of[NG_MAX_CHAINS];
  __shared__ int tmp[NG_T / 64];
  const int tid = threadIdx.x;
  const int W = p.W;

  for (int i = tid; i < W; i += NG_T) w[i] = p.window[i];
  if (tid < NG_MAX_CHAINS) chain_of[tid] = -1;
  // this thread's head candidate (node tid of the head part), read with the window
  const int head_nodes = 1 + 3 * p.levels;
  const int head_tok = tid >= 1 && tid < head_nodes && tid < p.T_max ? p.head[tid - 1] : -1;
  __syncthreads();
  const int root = w[W - 1];

  // occurrences i <= W - 4 of the root (the 4-gram lies in the window), in order
  int mine = 0;
#pragma unroll
  for (int s = 0; s < NG_SEG; ++s) {
    const int i = tid * NG_SEG + s;
    mine += (i <= W - 4 && w[i] == root) ? 1 : 0;
  }
  int M;
  int at = block_scan(mine, tmp, &M);
#pragma unroll
  for (int s = 0; s < NG_SEG; ++s) {
    const int i = tid * NG_SEG + s;
    if (i <= W - 4 && w[i] == root) {
      ka[at] = w[i + 1];
      kb[at] = w[i + 2];
      kc[at] = w[i + 3];
      ++at;
    }
  }
  __syncthreads();

  // first occurrence and count of each continuation (eight comparisons per
  // round; the first-occurrence scan stops at the round that finds a match)
  constexpr int R = 8;
  auto same = [&](int i, int a, int b, int c) { return ka[i] == a && kb[i] == b && kc[i] == c; };
  for (int j = tid; j < M; j += NG_T) {
    const int a = ka[j], b = kb[j], c = kc[j];
    bool first = true;
    for (int i0 = 0; i0 < j && first; i0 += R) {
#pragma unroll
      for (int u = 0; u < R; ++u) {
        const int i = i0 + u;
        if (i < j && same(i, a, b, c)) first = false;
      }
    }
    int n = 0;
    if (first)
      for (int i0 = j; i0 < M; i0 += R) {
#pragma unroll
        for (int u = 0; u < R; ++u) {
          const int i = i0 + u;
          n += (i < M && same(i, a, b, c)) ? 1 : 0;
        }
      }
    cnt[j] = n;   // n >= 1 exactly for first occurrences
  }
  __syncthreads();

  // distinct indices in order of first occurrence
  int nf = 0;
#pragma unroll
  for (int s = 0; s < NG_SEG; ++s) {
    const int j = tid * NG_SEG + s;
    nf += (j < M && cnt[j] > 0) ? 1 : 0;
  }
  int D;
  int q = block_scan(nf, tmp, &D);
#pragma unroll
  for (int s = 0; s < NG_SEG; ++s) {
    const int j = tid * NG_SEG + s;
    if (j < M) {
      const bool f = cnt[j] > 0;
      dq[j] = f ? q : -1;
      if (f) {
        rho[q] = splitmix64(p.seed, (u64)q);
        ++q;
      }
    }
  }
  __syncthreads();

  // keep: all, or the k smallest (rho, q); then the chain order among the kept
  const int k = p.k;
  const int kept = D < k ? D : k;
  for (int j = tid; j < M; j += NG_T) {
    const int qj = dq[j];
    if (qj < 0) continue;
    bool keep = true;
    if (D > k) {
      const u64 mine_r = rho[qj];
      int rank = 0;
      for (int r0 = 0; r0 < D; r0 += R) {
#pragma unroll
        for (int u = 0; u < R; ++u) {
          const int r = r0 + u;
          if (r < D) {
            const u64 x = rho[r];
            rank += (x < mine_r || (x == mine_r && r < qj)) ? 1 : 0;
          }
        }
      }
      keep = rank < k;
    }
    cnt[j] = keep ? cnt[j] : -cnt[j];   // kept first occurrences stay positive
  }
  __syncthreads();
  for (int j = tid; j < M; j += NG_T) {
    const int cj = cnt[j];
    if (cj <= 0) continue;
    int ord = 0;   // kept continuations before j: higher count, or equal count and earlier
    for (int i0 = 0; i0 < M; i0 += R) {
#pragma unroll
      for (int u = 0; u < R; ++u) {
        const int i = i0 + u;
        if (i < M) {
          const int ci = cnt[i];
          ord += (ci > cj || (ci == cj && i < j)) ? 1 : 0;
        }
      }
    }
    if (ord < NG_MAX_CHAINS) chain_of[ord] = j;
  }
  __syncthreads();

  // the tree, one thread per node slot
  const int L = p.levels;
  int T = head_nodes + 3 * kept;
  T = T < p.T_max ? T : p.T_max;
  if (tid < p.T_max) {
    int par = -1, tok = -1;
    if (tid == 0) {
      tok = root;
    } else if (tid < T && tid < head_nodes) {
      const int l = (tid - 1) / 3;
      tok = head_tok;
      par = l == 0 ? 0 : 3 * (l - 1) + 1;
    } else if (tid < T) {
      const int m = tid - head_nodes, c = m / 3, pos = m % 3;
      const int jc = chain_of[c];
      tok = pos == 0 ? ka[jc] : (pos == 1 ? kb[jc] : kc[jc]);
      par = pos == 0 ? 0 : tid - 1;
    }
    p.parent[tid] = par;
    p.node_token[tid] = tok;
  }
  if (tid == 0) {
    int placed = 0;
    for (int c = 0; c < kept; ++c) placed += (head_nodes + 3 * c < p.T_max) ? 1 : 0;
    p.info[0] = T;
    p.info[1] = placed;
    p.info[2] = D;
    p.info[3] = M;
  }
}

}  // namespace

hipError_t launch_ngram_tree(const NgramParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(ngram_tree_kernel, dim3(1), dim3(NG_T), 0, stream, p);
  return hipGetLastError();
}

}  // namespace ts
