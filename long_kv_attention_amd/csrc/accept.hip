// Tree acceptance and the post-acceptance KV commit for CDNA4 (gfx950).
//
// What is computed (TokenSwift summary §3.1 with Figure 2: the target model
// verifies the drafted tree in one pass and the longest valid draft is
// accepted, then the caches are updated; Appendix A: acceptance and rejection
// together keep the target's sampling distribution):
//   * a child c of node p continues a valid draft iff node_token[c] equals
//     target[p], the target model's token at p (its sample, or argmax);
//   * the accepted path ends at the deepest node whose edges from the root
//     are all valid (ties: the smaller node index); its nodes a_0 = 0 < ... <
//     a_m are committed and target[a_m] is the next token;
//   * commit: cache row n_ctx + k receives row n_ctx + a_k (k = 0..m) in every
//     layer and KV head, and the same rows are appended to the partial cache.
//
// Kernels:
//   accept  two waves, thread i = node i (up to 128): the target tokens to
//           LDS (one read of each), edge test, one ballot
//           per wave, validity as "no invalid edge among my ancestors" (two
//           ancestor words per node from the host), then a max of
//           (depth, -index) over both waves.
//   commit  grid (Hkv, layers, {K, V}): a workgroup loads its slice's m + 1
//           accepted rows into registers, waits for all of them, then stores
//           them (destination rows can be later source rows, so every load
//           precedes every store).
#include "ts_device.h"
#include "ts_internal.h"

#include <cstddef>
#include <type_traits>

namespace ts {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

static_assert(std::is_standard_layout<AcceptParams>::value, "kernarg offsets via offsetof");

__global__ __launch_bounds__(128) void accept_kernel(const AcceptParams p) {
  __shared__ u64 s_ok[2];
  __shared__ int s_key[2];
  __shared__ int32_t s_target[128];   // the target tokens, read once (ancestors' and the winner's come from here)
  const int i = threadIdx.x;
  const int wave = i >> 6;
  const bool in = i < p.T;
  // p is the kernel's only argument, so it starts the kernarg segment; the
  // per-node tables are read there with lane-varying indices
  const unsigned char* ka = (const unsigned char*)__builtin_amdgcn_kernarg_segment_ptr();
  const int32_t* par = reinterpret_cast<const int32_t*>(ka + offsetof(AcceptParams, parent));
  const u64* anc = reinterpret_cast<const u64*>(ka + offsetof(AcceptParams, anc));
  const int pi = in && i > 0 ? par[i] : 0;   // the host checked 0 <= parent[i] < i
  const int32_t tok = in ? p.node_token[i] : 0;
  if (in) s_target[i] = p.target[i];
  __syncthreads();
  const bool ok = in && (i == 0 || tok == s_target[pi]);
  const u64 okm = __ballot(ok);
  if ((i & 63) == 0) s_ok[wave] = okm;
  __syncthreads();
  const u64 ok0 = s_ok[0], ok1 = s_ok[1];
  const u64 m0 = in ? anc[2 * i] : 0ull, m1 = in ? anc[2 * i + 1] : 0ull;
  const bool valid = in && (m0 & ~ok0) == 0ull && (m1 & ~ok1) == 0ull;
  const int depth = __popcll(m0) + __popcll(m1) - 1;
  const int wkey = wave_reduce(valid ? (depth << 8) | (255 - i) : -1, OpMaxI());
  if ((i & 63) == 0) s_key[wave] = wkey;
  __syncthreads();
  const int key = s_key[0] > s_key[1] ? s_key[0] : s_key[1];   // node 0 is always valid
  const int best = 255 - (key & 255);
  const u64 pa0 = anc[2 * best], pa1 = anc[2 * best + 1];
  const int n = __popcll(pa0) + __popcll(pa1);
  if (i == 0) {
    p.result[0] = n;
    p.result[1] = s_target[best];
  }
  if (in) {
    const bool on = i < 64 ? ((pa0 >> i) & 1ull) != 0ull : ((pa1 >> (i - 64)) & 1ull) != 0ull;
    if (on) {
      const int rank = i < 64 ? __popcll(pa0 & ((1ull << i) - 1ull))
                              : __popcll(pa0) + __popcll(pa1 & ((1ull << (i - 64)) - 1ull));
      p.result[2 + rank] = i;
    }
    if (i >= n) p.result[2 + i] = -1;
  }
}

constexpr int CT = 256;   // threads per commit workgroup
constexpr int CPT = 8;    // 16-byte chunks per thread: 128 rows x 16 chunks (d = 128)

__global__ __launch_bounds__(CT) void commit_kernel(const CommitParams p) {
  const int g = blockIdx.x;
  const int layer = blockIdx.y;
  const bool is_v = blockIdx.z == 1;
  const int tid = threadIdx.x;
  const int nch = p.d / 8;
  int n = p.result[0];
  n = n < 1 ? 1 : (n > p.T ? p.T : n);   // a foreign buffer cannot push the copies out of range
  const int64_t off = (int64_t)layer * p.s_layer + (int64_t)g * p.s_head;
  uint16_t* base = (is_v ? p.v : p.k) + off;
  // the path entries, then the rows, each batch in flight together: items past
  // n * nch read clamped, valid entries and rows and store nothing (the
  // compiler would otherwise wait after each guarded load)
  int a[CPT];
#pragma unroll
  for (int it = 0; it < CPT; ++it) {
    const int r = (tid + it * CT) / nch;
    a[it] = p.result[2 + (r < p.T ? r : p.T - 1)];
  }
  u32x4 buf[CPT];
#pragma unroll
  for (int it = 0; it < CPT; ++it) {
    const int c = (tid + it * CT) % nch;
    const int ar = a[it] < 0 ? 0 : (a[it] >= p.T ? p.T - 1 : a[it]);
    buf[it] = *reinterpret_cast<const u32x4*>(base + (int64_t)(p.n_ctx + ar) * p.s_pos + c * 8);
  }
  __syncthreads();   // every source row is read before any row is overwritten
  uint16_t* pbase = p.k_part ? (is_v ? p.v_part : p.k_part) + (int64_t)layer * p.sp_layer + (int64_t)g * p.sp_head
                             : nullptr;
#pragma unroll
  for (int it = 0; it < CPT; ++it) {
    const int idx = tid + it * CT;
    if (idx < n * nch) {
      const int r = idx / nch, c = idx % nch;
      *reinterpret_cast<u32x4*>(base + (int64_t)(p.n_ctx + r) * p.s_pos + c * 8) = buf[it];
      if (pbase) *reinterpret_cast<u32x4*>(pbase + (int64_t)(p.n_part + r) * p.sp_pos + c * 8) = buf[it];
    }
  }
}

static_assert(CT * CPT >= 128 * 16, "one pass covers 128 rows of 16 chunks");

}  // namespace

hipError_t launch_accept(const AcceptParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(accept_kernel, dim3(1), dim3(128), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_commit(const CommitParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(commit_kernel, dim3(p.Hkv, p.layers, 2), dim3(CT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace ts
