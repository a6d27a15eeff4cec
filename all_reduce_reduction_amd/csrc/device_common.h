// device_common.h -- element types, reduction operators and 16-byte vector
// access for the gfx950 kernels.
//
// Arithmetic ("Inside NCCL all-reduce", section "What all-reduce
// promises": sum, prod, min, max, avg; avg pre-scales floating-point
// contributions by 1/n as they are read and divides integer sums once at
// the end):
//   - fp16/bf16 are widened exactly to fp32 in VGPRs, accumulated in fp32
//     and rounded once, to nearest even, when the result is written;
//   - int32 sum/prod wrap modulo 2^32 (unsigned arithmetic);
//   - min/max keep the accumulator unless the new operand is strictly
//     smaller/larger: acc = (b < a) ? b : a.
// The library is compiled with -ffp-contract=off so a multiply followed by
// an add is never fused: each fp32 operation rounds on its own.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "simar.h"

namespace simar {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int DT> struct Ty;
template <> struct Ty<SIM_INT32> { typedef int32_t S; typedef int32_t A; static constexpr int E = 4; };
template <> struct Ty<SIM_FP32>  { typedef float S;   typedef float A;   static constexpr int E = 4; };
template <> struct Ty<SIM_FP16>  { typedef uint16_t S; typedef float A;  static constexpr int E = 2; };
template <> struct Ty<SIM_BF16>  { typedef uint16_t S; typedef float A;  static constexpr int E = 2; };

// elements per 16-byte vector of storage
template <int DT> constexpr int epv() { return 16 / Ty<DT>::E; }

// ---- 16-bit codecs ----------------------------------------------------------
// The fp32 value is made opaque to the optimiser around each 16-bit
// conversion.  Otherwise gfx950 instruction selection folds a final fp32
// multiply or add together with the narrowing (or a widening together with
// the next multiply) into one mixed-precision FMA with a +0 addend: that
// rounds once instead of twice and turns -0 into +0, so the result would no
// longer be "fp32 arithmetic, then one RNE narrowing".  The empty asm emits
// no instruction.
__device__ __forceinline__ float opaque(float f) {
  asm("" : "+v"(f));
  return f;
}
__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  return opaque((float)__builtin_bit_cast(_Float16, (uint16_t)h));   // exact widening
}
__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)opaque(f));  // RNE (default mode)
}
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
  return __builtin_bit_cast(float, h << 16);                 // exact widening
}
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)opaque(f));   // RNE
}

// storage bits -> accumulator value (widen; no avg scaling)
template <int DT> __device__ __forceinline__ typename Ty<DT>::A widen_bits(uint32_t bits);
template <> __device__ __forceinline__ int32_t widen_bits<SIM_INT32>(uint32_t b) { return (int32_t)b; }
template <> __device__ __forceinline__ float widen_bits<SIM_FP32>(uint32_t b) { return __builtin_bit_cast(float, b); }
template <> __device__ __forceinline__ float widen_bits<SIM_FP16>(uint32_t b) { return f16_bits_to_f32(b & 0xffffu); }
template <> __device__ __forceinline__ float widen_bits<SIM_BF16>(uint32_t b) { return bf16_bits_to_f32(b & 0xffffu); }

// accumulator value -> storage bits (RNE for 16-bit)
template <int DT> __device__ __forceinline__ uint32_t narrow_bits(typename Ty<DT>::A v);
template <> __device__ __forceinline__ uint32_t narrow_bits<SIM_INT32>(int32_t v) { return (uint32_t)v; }
template <> __device__ __forceinline__ uint32_t narrow_bits<SIM_FP32>(float v) { return __builtin_bit_cast(uint32_t, v); }
template <> __device__ __forceinline__ uint32_t narrow_bits<SIM_FP16>(float v) { return f32_to_f16_bits(v); }
template <> __device__ __forceinline__ uint32_t narrow_bits<SIM_BF16>(float v) { return f32_to_bf16_bits(v); }

// ---- reduction operators ------------------------------------------------------
template <int DT, int OP> struct Op {
  typedef typename Ty<DT>::A A;
  // a contribution as it is read: fp avg scales by fp32(1/p)
  static __device__ __forceinline__ A pre(A x, float inv_p) {
    if constexpr (OP == SIM_AVG && DT != SIM_INT32) return x * inv_p;
    else return x;
  }
  // acc (+) b
  static __device__ __forceinline__ A comb(A a, A b) {
    if constexpr (DT == SIM_INT32) {
      if constexpr (OP == SIM_SUM || OP == SIM_AVG) return (int32_t)((uint32_t)a + (uint32_t)b);
      else if constexpr (OP == SIM_PROD) return (int32_t)((uint32_t)a * (uint32_t)b);
      else if constexpr (OP == SIM_MIN) return (b < a) ? b : a;
      else return (b > a) ? b : a;
    } else {
      if constexpr (OP == SIM_SUM || OP == SIM_AVG) return a + b;
      else if constexpr (OP == SIM_PROD) return a * b;
      else if constexpr (OP == SIM_MIN) return (b < a) ? b : a;
      else return (b > a) ? b : a;
    }
  }
  // the fix-up where a chunk completes: int avg divides once (truncating)
  static __device__ __forceinline__ A post(A v, int p) {
    if constexpr (OP == SIM_AVG && DT == SIM_INT32) return v / p;
    else return v;
  }
};

// ---- 16-byte vectors -----------------------------------------------------------
// Bulk data is touched once per call, so loads and stores are streaming
// (nontemporal) by default: they should not evict other data from L2/MALL.
#ifndef SIMAR_LOAD_NT
#define SIMAR_LOAD_NT 1
#endif
#ifndef SIMAR_STORE_NT
#define SIMAR_STORE_NT 1
#endif
// Every buffer is device-visible global memory: the accesses are typed as
// such (global_load/store, with a scalar base where the address allows it)
// rather than generic flat accesses -- pointers read from memory, such as the
// pointer table's, would otherwise stay generic.
typedef __attribute__((address_space(1))) const u32x4 gconst_u32x4;
typedef __attribute__((address_space(1))) u32x4 g_u32x4;
__device__ __forceinline__ u32x4 ld16(const void* base, int64_t byte_off) {
  gconst_u32x4* p = (gconst_u32x4*)((const char*)base + byte_off);
#if SIMAR_LOAD_NT
  return __builtin_nontemporal_load(p);
#else
  return *p;
#endif
}
__device__ __forceinline__ void st16(void* base, int64_t byte_off, u32x4 v) {
  g_u32x4* p = (g_u32x4*)((char*)base + byte_off);
#if SIMAR_STORE_NT
  __builtin_nontemporal_store(v, p);
#else
  *p = v;
#endif
}

// The same access split into a workgroup-uniform byte offset and a 32-bit
// per-lane offset: base + uoff is computed in scalar registers and the lane
// offset rides in one VGPR shared by every operand (the global_load/store
// form with a scalar base), instead of a 64-bit address pair per operand.
__device__ __forceinline__ u32x4 ld16u(const void* base, int64_t uoff, uint32_t lane_off) {
  return ld16((const char*)base + uoff, (int64_t)lane_off);
}
__device__ __forceinline__ void st16u(void* base, int64_t uoff, uint32_t lane_off, u32x4 v) {
  st16((char*)base + uoff, (int64_t)lane_off, v);
}
// Hide a per-lane offset's derivation from the optimiser for one loop
// iteration, so it is not folded into loop-invariant 64-bit pointers (one
// VGPR pair per operand would cut the waves a SIMD can hold).
__device__ __forceinline__ uint32_t lane_offset(uint32_t off) {
  asm volatile("" : "+v"(off));
  return off;
}

// Unpack one 16-byte storage vector into EPV accumulator values.
template <int DT>
__device__ __forceinline__ void unpack(u32x4 v, typename Ty<DT>::A* out) {
  if constexpr (Ty<DT>::E == 4) {
#pragma unroll
    for (int k = 0; k < 4; k++) out[k] = widen_bits<DT>(v[k]);
  } else {
#pragma unroll
    for (int k = 0; k < 4; k++) {
      out[2 * k] = widen_bits<DT>(v[k] & 0xffffu);
      out[2 * k + 1] = widen_bits<DT>(v[k] >> 16);
    }
  }
}

// Pack EPV accumulator values into one 16-byte storage vector.
template <int DT>
__device__ __forceinline__ u32x4 pack(const typename Ty<DT>::A* in) {
  u32x4 v;
  if constexpr (Ty<DT>::E == 4) {
#pragma unroll
    for (int k = 0; k < 4; k++) v[k] = narrow_bits<DT>(in[k]);
  } else {
#pragma unroll
    for (int k = 0; k < 4; k++) v[k] = narrow_bits<DT>(in[2 * k]) | (narrow_bits<DT>(in[2 * k + 1]) << 16);
  }
  return v;
}

// Where partial j sits in an accumulator-typed partial buffer.  A lane
// handles V elements per vector; for 16-bit types that is 8 partials of
// 4 bytes, 32 bytes, stored as two 16-byte halves.  Kept in element order,
// each 16-byte store instruction of a wave would write every other 16 bytes
// of a 2 KiB run, and the half-filled lines reach memory as separate
// partial writes.  So the partials of 16-bit types are laid out in blocks
// of 512 elements (one wave's 64 vectors) as [half][lane][4]: every store
// or load instruction of a wave covers one contiguous 1 KiB run.  32-bit
// types (one 16-byte vector per lane, partials sometimes kept in the
// outputs) stay in element order.  Buffers of 16-bit partials are sized in
// whole blocks of 512 elements.
template <int DT>
__device__ __forceinline__ int64_t part_pos(int64_t j) {
  if constexpr (Ty<DT>::E == 4) {
    return j;
  } else {
    const int w = (int)(j & 511);  // w = lane * 8 + k within the block
    return (j - w) + ((w & 4) << 6) + ((w >> 3) << 2) + (w & 3);
  }
}

// accumulator-typed partials: V values at element index idx (vector aligned)
template <int DT>
__device__ __forceinline__ void load_part(const void* base, int64_t idx, typename Ty<DT>::A* out) {
  constexpr int V = epv<DT>();
#pragma unroll
  for (int h = 0; h < V / 4; h++) {
    const u32x4 w = ld16(base, part_pos<DT>(idx + 4 * h) * 4);
#pragma unroll
    for (int k = 0; k < 4; k++) {
      // copy the lane out first: a bit cast applied directly to a vector
      // subscript reads element 0 with this compiler
      const uint32_t bits = w[k];
      out[4 * h + k] = __builtin_bit_cast(typename Ty<DT>::A, bits);
    }
  }
}
template <int DT>
__device__ __forceinline__ void store_part(void* base, int64_t idx, const typename Ty<DT>::A* in) {
  constexpr int V = epv<DT>();
#pragma unroll
  for (int h = 0; h < V / 4; h++) {
    u32x4 w;
#pragma unroll
    for (int k = 0; k < 4; k++) w[k] = __builtin_bit_cast(uint32_t, in[4 * h + k]);
    st16(base, part_pos<DT>(idx + 4 * h) * 4, w);
  }
}

// Scalar element access (ragged heads and tails).
template <int DT>
__device__ __forceinline__ typename Ty<DT>::A load_elem(const void* base, int64_t i) {
  if constexpr (Ty<DT>::E == 4) return widen_bits<DT>(((const uint32_t*)base)[i]);
  else return widen_bits<DT>(((const uint16_t*)base)[i]);
}
template <int DT>
__device__ __forceinline__ void store_elem(void* base, int64_t i, typename Ty<DT>::A v) {
  if constexpr (Ty<DT>::E == 4) ((uint32_t*)base)[i] = narrow_bits<DT>(v);
  else ((uint16_t*)base)[i] = (uint16_t)narrow_bits<DT>(v);
}

}  // namespace simar
