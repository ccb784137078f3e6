// Device helpers shared by the kernels of this library (gfx950).
#pragma once

#include <hip/hip_runtime.h>

namespace ts {

typedef unsigned long long u64;

// Workgroup barrier for LDS only: the kernels that use it never read global
// memory that another thread of the workgroup wrote in the same launch, so
// outstanding global stores need not drain at every barrier (__syncthreads
// would wait for them).
__device__ inline void bar() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ inline u64 lanemask_lt() { return (1ull << (threadIdx.x & 63)) - 1ull; }

// ---- wave reductions without LDS: DPP rotations inside each 16-lane row,
// then the gfx950 row-pair and half swaps (v_permlane16/32_swap: with both
// operands holding x, one result holds rows 0,0,2,2 and the other 1,1,3,3, and
// likewise for the halves). Integer results are the same in every lane; float
// sums can differ between lanes in the last bit, so callers use lane 0's. ----
template <int CTRL>
__device__ inline unsigned int dpp32(unsigned int x) {
  return (unsigned int)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xf, 0xf, false);
}
template <typename T>
__device__ inline void to_words(T x, unsigned int (&w)[sizeof(T) / 4]) { __builtin_memcpy(w, &x, sizeof(T)); }
template <typename T>
__device__ inline T from_words(const unsigned int (&w)[sizeof(T) / 4]) {
  T x;
  __builtin_memcpy(&x, w, sizeof(T));
  return x;
}
template <int CTRL, typename T>
__device__ inline T dpp_t(T x) {
  unsigned int w[sizeof(T) / 4];
  to_words(x, w);
#pragma unroll
  for (unsigned int& v : w) v = dpp32<CTRL>(v);
  return from_words<T>(w);
}
template <bool HALVES, typename T>
__device__ inline void swap_t(T x, T& a, T& b) {
  unsigned int w[sizeof(T) / 4], wa[sizeof(T) / 4], wb[sizeof(T) / 4];
  to_words(x, w);
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 4); ++i) {
    const auto r = HALVES ? __builtin_amdgcn_permlane32_swap(w[i], w[i], false, false)
                          : __builtin_amdgcn_permlane16_swap(w[i], w[i], false, false);
    wa[i] = r[0];
    wb[i] = r[1];
  }
  a = from_words<T>(wa);
  b = from_words<T>(wb);
}
template <typename T, typename Op>
__device__ inline T wave_reduce(T x, Op op) {
  x = op(x, dpp_t<0x128>(x));   // row_ror:8
  x = op(x, dpp_t<0x124>(x));   // row_ror:4
  x = op(x, dpp_t<0x122>(x));   // row_ror:2
  x = op(x, dpp_t<0x121>(x));   // row_ror:1
  T a, b;
  swap_t<false>(x, a, b);
  x = op(a, b);
  swap_t<true>(x, a, b);
  return op(a, b);
}
struct OpMax { __device__ float operator()(float a, float b) const { return fmaxf(a, b); } };
struct OpAdd { template <typename T> __device__ T operator()(T a, T b) const { return a + b; } };
struct OpMinU { __device__ u64 operator()(u64 a, u64 b) const { return a < b ? a : b; } };
struct OpMaxI { __device__ int operator()(int a, int b) const { return a > b ? a : b; } };

}  // namespace ts
