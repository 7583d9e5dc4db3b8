// Shared device/host definitions of libmuonstep (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "muon_step.h"
#include "common_host.hpp"

#define MUON_LDS __attribute__((address_space(3)))

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));

namespace muon {

// Per-problem descriptor (one Newton-Schulz problem = a matrix or a split block).
// A problem's elements, in stored (row-major) order, have local flat indices
// e in [0, rows * cols). Momentum, gradient and update_out element e sits at
// src_off + e; the step applies its update to e in [lo, hi) only, at params
// index p_base + e (the whole problem at src_off + e for an ordinary step; a
// window of a matrix that straddles a parameter partition otherwise).
// Block element (r, c) of a problem (stored orientation) is at src_off + r * ld +
// c in grads / momentum / update_out and at p_base + r * ld + c in params; its
// local index r * ld + c is applied when lo <= index < hi.
struct ProblemDesc {
  int64_t src_off;
  int64_t p_base;
  int64_t lo, hi;
  int32_t transposed;  // 1: stored rows x cols with rows > cols, canonical = stored^T
  int32_t ld;          // row pitch in elements (the matrix's cols)
  int32_t w;           // stored width (block cols); ld == w: the block is contiguous
  int32_t pad;
};

// ---------------------------------------------------------------------------
// element conversions (round to nearest even, the hardware default)

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return static_cast<__bf16>(x); }
template <> __device__ __forceinline__ _Float16 from_f32<_Float16>(float x) { return static_cast<_Float16>(x); }

template <typename T> __device__ __forceinline__ float to_f32(T x) { return static_cast<float>(x); }

// x as a materialised fp32 value: a conversion that follows rounds this value,
// instead of being merged with the arithmetic that produced x into a single
// rounding (which the compiler does for fp16 results in some kernels and not in
// others). Every kernel that stores an iterate rounds it this way.
__device__ __forceinline__ float keep_f32(float x) {
  asm volatile("" : "+v"(x));
  return x;
}

// N values (N even) rounded to T, nearest even, as from_f32 rounds them; the
// 16-bit types convert two per instruction
template <typename T, int N>
__device__ __forceinline__ void rne(const float (&v)[N], T (&o)[N]) {
  static_assert(N % 2 == 0, "pairs");
  if constexpr (sizeof(T) == 2) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef T t2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int p = 0; p < N / 2; ++p) {
      const f2 x = {keep_f32(v[2 * p]), keep_f32(v[2 * p + 1])};
      const t2 y = __builtin_convertvector(x, t2);
      o[2 * p] = y[0];
      o[2 * p + 1] = y[1];
    }
  } else {
#pragma unroll
    for (int e = 0; e < N; ++e) o[e] = from_f32<T>(keep_f32(v[e]));
  }
}

__device__ __forceinline__ unsigned short bf16_bits(float x) {
  __bf16 b = static_cast<__bf16>(x);
  return __builtin_bit_cast(unsigned short, b);
}

__device__ __forceinline__ float bf16_bits_to_f32(unsigned short u) {
  return __uint_as_float(static_cast<uint32_t>(u) << 16);
}

__device__ __forceinline__ float f16_bits_to_f32(unsigned short u) {
  return static_cast<float>(__builtin_bit_cast(_Float16, u));
}

// grad element -> float (grad dtype chosen at run time per launch template)
template <int GDT> __device__ __forceinline__ float grad_to_f32(const void* g, int64_t i);
template <> __device__ __forceinline__ float grad_to_f32<MUON_DTYPE_F32>(const void* g, int64_t i) {
  return static_cast<const float*>(g)[i];
}
template <> __device__ __forceinline__ float grad_to_f32<MUON_DTYPE_BF16>(const void* g, int64_t i) {
  return bf16_bits_to_f32(static_cast<const unsigned short*>(g)[i]);
}
template <> __device__ __forceinline__ float grad_to_f32<MUON_DTYPE_F16>(const void* g, int64_t i) {
  return f16_bits_to_f32(static_cast<const unsigned short*>(g)[i]);
}

// 4 consecutive grad elements (8-byte aligned for 16-bit types, 16-byte for f32).
// Gradients are read exactly once per step: non-temporal loads keep them from
// displacing cached data (also in load_grad2).
template <int GDT> __device__ __forceinline__ void load_grad4(const void* g, int64_t i, float (&o)[4]);
template <> __device__ __forceinline__ void load_grad4<MUON_DTYPE_F32>(const void* g, int64_t i, float (&o)[4]) {
  const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(static_cast<const float*>(g) + i));
  o[0] = a[0]; o[1] = a[1]; o[2] = a[2]; o[3] = a[3];
}
template <> __device__ __forceinline__ void load_grad4<MUON_DTYPE_BF16>(const void* g, int64_t i, float (&o)[4]) {
  const u16x4 v = __builtin_nontemporal_load(reinterpret_cast<const u16x4*>(static_cast<const unsigned short*>(g) + i));
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = bf16_bits_to_f32(v[e]);
}
template <> __device__ __forceinline__ void load_grad4<MUON_DTYPE_F16>(const void* g, int64_t i, float (&o)[4]) {
  const u16x4 v = __builtin_nontemporal_load(reinterpret_cast<const u16x4*>(static_cast<const unsigned short*>(g) + i));
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = f16_bits_to_f32(v[e]);
}

// 2 consecutive grad elements (4-byte aligned for 16-bit types, 8-byte for f32)
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
template <int GDT> __device__ __forceinline__ void load_grad2(const void* g, int64_t i, float (&o)[2]);
template <> __device__ __forceinline__ void load_grad2<MUON_DTYPE_F32>(const void* g, int64_t i, float (&o)[2]) {
  const f32x2 a = __builtin_nontemporal_load(reinterpret_cast<const f32x2*>(static_cast<const float*>(g) + i));
  o[0] = a[0]; o[1] = a[1];
}
template <> __device__ __forceinline__ void load_grad2<MUON_DTYPE_BF16>(const void* g, int64_t i, float (&o)[2]) {
  const u16x2 v = __builtin_nontemporal_load(reinterpret_cast<const u16x2*>(static_cast<const unsigned short*>(g) + i));
  o[0] = bf16_bits_to_f32(v[0]); o[1] = bf16_bits_to_f32(v[1]);
}
template <> __device__ __forceinline__ void load_grad2<MUON_DTYPE_F16>(const void* g, int64_t i, float (&o)[2]) {
  const u16x2 v = __builtin_nontemporal_load(reinterpret_cast<const u16x2*>(static_cast<const unsigned short*>(g) + i));
  o[0] = f16_bits_to_f32(v[0]); o[1] = f16_bits_to_f32(v[1]);
}

// ---------------------------------------------------------------------------
// wave / block reductions (fixed order: deterministic)

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace muon
