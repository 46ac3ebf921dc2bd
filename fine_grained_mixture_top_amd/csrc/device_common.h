// Device-side helpers shared by the MoE kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint16_t bf16_t;  // bf16 storage (bit pattern)
typedef __bf16 bf16x8_v __attribute__((ext_vector_type(8)));
typedef float f32x4_v __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;

__device__ __forceinline__ float bf2f(bf16_t h) { return __uint_as_float((uint32_t)h << 16); }

typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest even (NaN kept quiet): gfx950's conversion
// instruction (v_cvt_pk_bf16_f32, two values per instruction).
__device__ __forceinline__ bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

// two values -> one packed word (a in the low half)
__device__ __forceinline__ uint32_t f2bf2(float a, float b) {
  const bf16x2_v v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int VEC = 4;   // elements per 16-byte vector
  static constexpr int BK = 32;   // k elements per main-loop step (128 bytes)
  __device__ static float to_f(float v) { return v; }
  __device__ static float from_f(float v) { return v; }
};
template <> struct Elem<bf16_t> {
  static constexpr int VEC = 8;
  static constexpr int BK = 64;
  __device__ static float to_f(bf16_t v) { return bf2f(v); }
  __device__ static bf16_t from_f(float v) { return f2bf(v); }
};

// Round a value through the storage type (identity for fp32).
template <typename T> __device__ __forceinline__ float through(float v) {
  return Elem<T>::to_f(Elem<T>::from_f(v));
}

// logistic sigmoid with the hardware exponential and reciprocal (about one
// ulp each; the forward and the backward's recomputation share this code)
__device__ __forceinline__ float sigmoidf_(float g) { return __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

// Largest i in [0, n) with a[i] <= v (a non-decreasing, a[0] <= v).
__device__ __forceinline__ int upper_index(const int32_t* a, int n, int v) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (a[mid] <= v) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Sum over the 16 lanes that share lane/16 (xor butterfly inside a row of 16).
__device__ __forceinline__ float sum16(float v) {
  v += __shfl_xor(v, 1, 64);
  v += __shfl_xor(v, 2, 64);
  v += __shfl_xor(v, 4, 64);
  v += __shfl_xor(v, 8, 64);
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// ---------------------------------------------------------------------------
// LDS staging next to buffer -> LDS loads in flight.
//
// The compiler orders LDS accesses against the loads that write LDS
// directly (buffer_load ... lds) by waiting for all of them (vmcnt(0)):
//  * before a __syncthreads(), whose workgroup fence covers LDS, whenever
//    such a load may still be outstanding;
//  * before a ds_read / ds_write that carries no type-based alias
//    information, e.g. one through HIP's uint2 / uint4 / float4 structs.
// The kernels that stream operand stages that way keep several stages in
// flight on purpose and wait for exactly the stage they read with explicit
// vmcnt waits; the LDS they write with ds_write (epilogue staging) never
// overlaps a stage still being loaded.  So they use lds_sync() and the
// typed accesses below, and those drains do not happen.
// ---------------------------------------------------------------------------

// Workgroup barrier for LDS: every wave's own ds_read / ds_write complete
// (lgkmcnt(0)), then all waves meet; loads into LDS still in flight are left
// alone.  The empty asm statements keep the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void lds_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt at their maximum
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

typedef uint32_t u32x2_lv __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_lv __attribute__((ext_vector_type(4)));

// 8- and 16-byte LDS accesses through clang vector types
__device__ __forceinline__ void lds_st8(void* p, uint2 v) { *reinterpret_cast<u32x2_lv*>(p) = u32x2_lv{v.x, v.y}; }
__device__ __forceinline__ uint4 lds_ld16(const void* p) {
  const u32x4_lv v = *reinterpret_cast<const u32x4_lv*>(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void lds_st_f4(void* p, float a, float b, float c, float d) {
  *reinterpret_cast<f32x4_v*>(p) = f32x4_v{a, b, c, d};
}
__device__ __forceinline__ f32x4_v lds_ld_f4(const void* p) { return *reinterpret_cast<const f32x4_v*>(p); }

// Map a workgroup id so that consecutive virtual ids land on the same XCD.
// Workgroups are dispatched round-robin over the 8 XCDs, so physical id b runs
// on XCD b % 8; virtual id (b % 8) * (G / 8) + b / 8 gives each XCD one
// contiguous run of G / 8 virtual ids (G a multiple of 8).
__device__ __forceinline__ int xcd_virtual_id(int b, int G) {
  if ((G & 7) != 0) return b;
  return (b & 7) * (G >> 3) + (b >> 3);
}

}  // namespace moe
