// Element-wise access to optimizer state (W, M, G and the buffers built from them) of
// one element type T, bf16, f16 or fp32, in 16-byte chunks: 8 elements of a 16-bit
// type or 4 fp32 elements.  Shared by the Dion3 and Muon element-wise kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace gns {

// Raw bits of element i of a 16-byte chunk of T, and the chunk holding given element
// bits.
template <class T>
__device__ __forceinline__ uint32_t elem_bits(const uint4& c, int i) {
  const uint32_t* w = reinterpret_cast<const uint32_t*>(&c);
  if constexpr (T::kBytes == 4) return w[i];
  else return (i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xffffu);
}
template <class T>
__device__ __forceinline__ uint4 pack_bits(const uint32_t (&b)[T::kPerChunk]) {
  uint4 c;
  uint32_t* w = reinterpret_cast<uint32_t*>(&c);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (T::kBytes == 4) w[i] = b[i];
    else w[i] = b[2 * i] | (b[2 * i + 1] << 16);
  }
  return c;
}
// An fp32 result rounded to T (bits).  For f16 the value first passes through an empty
// asm statement: without it the compiler may merge the fp32 operation that produced it
// and the conversion into one mixed-precision instruction (v_fma_mix*), which rounds
// the exact result once to f16 instead of rounding the fp32 result, and differs from
// that on ties.
template <class T>
__device__ __forceinline__ uint32_t round_to(float x) {
  if constexpr (T::kId == GNS_F16) asm volatile("" : "+v"(x));
  return T::from_f32(x);
}

// The elements of a chunk widened to fp32, and the chunk of fp32 values each rounded
// once to T.
template <class T>
__device__ __forceinline__ void unpack(const uint4& c, float (&v)[T::kPerChunk]) {
#pragma unroll
  for (int i = 0; i < T::kPerChunk; ++i) v[i] = T::to_f32(elem_bits<T>(c, i));
}
template <class T>
__device__ __forceinline__ uint4 pack(const float (&v)[T::kPerChunk]) {
  uint32_t b[T::kPerChunk];
#pragma unroll
  for (int i = 0; i < T::kPerChunk; ++i) b[i] = round_to<T>(v[i]);
  return pack_bits<T>(b);
}

template <class T>
__device__ __forceinline__ uint4* row_chunks(void* base, long long elems) {
  return reinterpret_cast<uint4*>(static_cast<uint8_t*>(base) + (size_t)elems * T::kBytes);
}
template <class T>
__device__ __forceinline__ const uint4* row_chunks(const void* base, long long elems) {
  return reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(base) + (size_t)elems * T::kBytes);
}

// The launchers take the state type at run time: call f with a tag of that type.
template <class F>
hipError_t with_state_type(gns_dtype dt, F&& f) {
  switch (dt) {
    case GNS_BF16: return f(TBF16{});
    case GNS_F16: return f(TF16{});
    case GNS_F32: return f(TF32{});
  }
  return hipErrorInvalidValue;
}

}  // namespace gns
