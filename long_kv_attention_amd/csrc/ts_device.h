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

// The value lane `src` holds, in every lane (src wave-uniform), VALU only.
__device__ inline unsigned int lane_value(unsigned int v, int src) {
  return (unsigned int)__builtin_amdgcn_readlane((int)v, src);   // readlane's int, widened unsigned
}
__device__ inline u64 lane_value(u64 v, int src) {
  return (u64)lane_value((unsigned int)v, src) | ((u64)lane_value((unsigned int)(v >> 32), src) << 32);
}

// Inclusive prefix sum over the 64 lanes of a wave, with no LDS round trip:
// Hillis-Steele steps inside each 16-lane row by DPP row shifts (1, 2, 4, 8;
// a lane shifted in from outside its row adds 0), then each lane adds the
// totals of the rows below it, read from lanes 15, 31 and 47. Every lane of
// the wave must be active. Exact for integers (the order of the additions
// does not matter).
template <int CTRL>
__device__ inline unsigned int dpp_zero(unsigned int v) {
  return (unsigned int)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}
template <int CTRL>
__device__ inline u64 dpp_zero(u64 v) {
  return (u64)dpp_zero<CTRL>((unsigned int)v) | ((u64)dpp_zero<CTRL>((unsigned int)(v >> 32)) << 32);
}
template <typename T>
__device__ inline T wave_incl_scan_t(T x) {
  x += dpp_zero<0x111>(x);   // row_shr:1
  x += dpp_zero<0x112>(x);   // row_shr:2
  x += dpp_zero<0x114>(x);   // row_shr:4
  x += dpp_zero<0x118>(x);   // row_shr:8
  const T r0 = lane_value(x, 15), r1 = lane_value(x, 31), r2 = lane_value(x, 47);
  const unsigned int lane = threadIdx.x & 63;
  return x + (lane >= 16 ? r0 : T(0)) + (lane >= 32 ? r1 : T(0)) + (lane >= 48 ? r2 : T(0));
}
__device__ inline unsigned int wave_incl_scan(unsigned int x) { return wave_incl_scan_t(x); }
__device__ inline u64 wave_incl_scan(u64 x) { return wave_incl_scan_t(x); }
__device__ inline int wave_incl_scan(int x) { return (int)wave_incl_scan_t((unsigned int)x); }

// x[l] + x[l ^ M] in every lane l, VALU only: the gfx950 row swaps for M = 16
// and 32 (with both operands holding x, the two results are the two lanes'
// values), a DPP row rotation by 8 inside 16-lane rows for M = 8. Float
// addition is commutative, so both lanes of a pair get the same bits.
template <int M>
__device__ inline float xor_add(float x) {
  if constexpr (M == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  } else if constexpr (M == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  } else {
    static_assert(M == 8, "xor distances 8, 16, 32");
    return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false));
  }
}

#define LDS_AS __attribute__((address_space(3)))

// LDS byte address of a __shared__ object (the M0 value of an LDS copy).
__device__ inline unsigned int lds_offset(const void* p) {
  return (unsigned int)(uintptr_t)(const LDS_AS void*)p;
}

// Order-preserving map from float to uint32 (a larger float gives a larger
// key; -0 sorts just below +0): the usual radix-sort key of IEEE floats.
__device__ inline unsigned int f2key(float f) {
  const unsigned int u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer resource (gfx9 layout): 48-bit base, stride 0, num_records bytes.
// Reads at offsets >= num_records are out of range and do not touch memory.
__device__ inline i32x4 buffer_desc(const void* base, unsigned int num_records) {
  const unsigned long long b = reinterpret_cast<unsigned long long>(base);
  return i32x4{(int)(unsigned int)b, (int)((unsigned int)(b >> 32) & 0xffffu), (int)num_records, 0x00020000};
}

// One wave-wide asynchronous copy global -> LDS (16 B per lane): lane l's 16
// bytes come from the buffer at byte offset off + soff (soff wave-uniform)
// and land at LDS byte lds_off + 16 * l. The compiler does not see the LDS
// write; callers order it with explicit vmcnt waits and barriers. One wait
// state separates the M0 write from the load that reads it.
__device__ inline void dma16(i32x4 desc, unsigned int off, unsigned int soff, unsigned int lds_off) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(__builtin_amdgcn_readfirstlane(lds_off)), "v"(off), "s"(desc),
                  "s"(__builtin_amdgcn_readfirstlane(soff)) : "memory", "m0");
}

// The same with no scalar offset (one instruction less to set up).
__device__ inline void dma16(i32x4 desc, unsigned int off, unsigned int lds_off) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(__builtin_amdgcn_readfirstlane(lds_off)), "v"(off), "s"(desc) : "memory", "m0");
}

// The same copy with the non-temporal cache policy, for data streamed once
// (the K/V cache): measured on an LDS-copy ring over a 100K-row cache, it
// streams at 6.8-7.0 TB/s instead of 5.8-6.1 TB/s with the default policy.
__device__ inline void dma16_nt(i32x4 desc, unsigned int off, unsigned int soff, unsigned int lds_off) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds"
               :: "s"(__builtin_amdgcn_readfirstlane(lds_off)), "v"(off), "s"(desc),
                  "s"(__builtin_amdgcn_readfirstlane(soff)) : "memory", "m0");
}

// Wait until at most N vector-memory operations of this wave are in flight
// (and every LDS operation is done).
template <int N>
__device__ inline void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" :: "n"(N) : "memory");
}

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
