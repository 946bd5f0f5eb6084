// Device helpers for the gfx950 kernels: storage-type traits, 16-byte vector
// loads, and wave-level reductions built on DPP row permutations.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace bsp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Storage-type traits: conversion to and from fp32.
template <typename T> struct Traits;
template <> struct Traits<float> {
  static __device__ __forceinline__ float to_f(float x) { return x; }
  static __device__ __forceinline__ float from_f(float x) { return x; }
};
template <> struct Traits<_Float16> {
  static __device__ __forceinline__ float to_f(_Float16 x) { return (float)x; }
  static __device__ __forceinline__ _Float16 from_f(float x) { return (_Float16)x; }
};
template <> struct Traits<__bf16> {
  static __device__ __forceinline__ float to_f(__bf16 x) { return (float)x; }
  static __device__ __forceinline__ __bf16 from_f(float x) { return (__bf16)x; }
};

// Buffer resource over [base, base + bytes) for raw (stride 0) dword buffer
// operations: an access past the end reads 0 and writes nothing. Word 3 selects
// the 32-bit data format that untyped buffer loads and stores use on CDNA.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
// Cache-policy operand of a buffer load or store that is coherent across the
// whole device (the sc1 bit: the access is made at the device's coherence
// point, so data written by a workgroup on another XCD is seen).
constexpr int kCoherentAgent = 16;

// Store with the non-temporal hint. The fused beam step at one query block per
// wave writes its outputs and the current tokens' pool rows this way when they
// fit the L2s: a plain store leaves the line dirty in the XCD's L2, and at the
// end of a kernel every XCD writes its dirty lines back before the next kernel
// starts, so such a step paid for all of its writes after its last workgroup
// (0.6B-like step 41.3 -> 38.3 us per launch). The prefill, partial-state,
// merge and KV-write kernels measured slower with it and keep plain stores.
template <typename V>
__device__ __forceinline__ void stream_store(V* p, V v) { __builtin_nontemporal_store(v, p); }
// A non-temporal or a plain store, by a run-time flag. The two branches carry
// different (empty) asm markers before and after their store: with identical
// neighbours the compiler hoists or sinks the two stores into one and keeps
// it without the hint.
template <typename V>
__device__ __forceinline__ void store_maybe_stream(V* p, V v, bool stream) {
  if (stream) {
    asm volatile("; streaming store");
    __builtin_nontemporal_store(v, p);
    asm volatile("; streaming store done");
  } else {
    asm volatile("; store");
    *p = v;
    asm volatile("; store done");
  }
}

// 2^x on the transcendental unit (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// DPP move with a compile-time control word; every source lane is valid for
// the quad permutations and mirrors used here.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i inside each group of 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i inside each row of 16

// Sum / max over each row of 16 lanes; every lane of the row gets the result.
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_mov<kDppXor1>(x);
  x += dpp_mov<kDppXor2>(x);
  x += dpp_mov<kDppHalfMirror>(x);
  x += dpp_mov<kDppMirror>(x);
  return x;
}
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_mov<kDppXor1>(x));
  x = fmaxf(x, dpp_mov<kDppXor2>(x));
  x = fmaxf(x, dpp_mov<kDppHalfMirror>(x));
  x = fmaxf(x, dpp_mov<kDppMirror>(x));
  return x;
}

// Wave-uniform sum / max over all 64 lanes.
__device__ __forceinline__ float wave_sum(float x) {
  x = row16_sum(x);
  float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 0));
  float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 16));
  float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 32));
  float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 48));
  return (a + b) + (c + d);
}
__device__ __forceinline__ float wave_max(float x) {
  x = row16_max(x);
  float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 0));
  float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 16));
  float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 32));
  float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 48));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

// Exchange with lane (lane ^ 16) / (lane ^ 32) of the same wave.
__device__ __forceinline__ float xor16(float x) { return __shfl_xor(x, 16, 64); }
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

// Max / sum of the four lanes {l, l^16, l^32, l^48}, every one of them getting
// the same value. The permlane swaps hand each lane its partner's value in a
// single VALU operation (no LDS round trip): a swap of x with itself across
// 16-lane rows (or 32-lane halves) leaves x in one result register and the
// partner's x in the other, in an order that depends on the lane, so only
// order-free combinations (max, and the commutative sum of two terms) are taken.
// The halves are converted through by-value helpers: a bit cast applied
// directly to an element of the returned vector reads element 0.
__device__ __forceinline__ float u2f(unsigned u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ unsigned f2u(float f) { return __builtin_bit_cast(unsigned, f); }
__device__ __forceinline__ float max4x16(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(f2u(x), f2u(x), false, false);
  const unsigned a0 = a[0], a1 = a[1];
  x = fmaxf(u2f(a0), u2f(a1));
  const auto b = __builtin_amdgcn_permlane32_swap(f2u(x), f2u(x), false, false);
  const unsigned b0 = b[0], b1 = b[1];
  return fmaxf(u2f(b0), u2f(b1));
}
__device__ __forceinline__ float sum4x16(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(f2u(x), f2u(x), false, false);
  const unsigned a0 = a[0], a1 = a[1];
  x = u2f(a0) + u2f(a1);
  const auto b = __builtin_amdgcn_permlane32_swap(f2u(x), f2u(x), false, false);
  const unsigned b0 = b[0], b1 = b[1];
  return u2f(b0) + u2f(b1);
}

__device__ __forceinline__ void record_fault(int32_t* bits, int32_t* count, int32_t* first,
                                             int32_t bit, int32_t value) {
  // Vector-memory atomics on the caller's workspace.
  if (atomicAdd(count, 1) == 0) atomicExch(first, value);
  atomicOr(bits, bit);
}

}  // namespace bsp
