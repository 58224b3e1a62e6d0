// Device-side building blocks shared by the gfx950 kernels of libgns:
// element types, conversions, 16-byte LDS chunk swizzle and the MFMA step.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/gns.h"

namespace gns {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Round to nearest even; NaN -> quiet NaN.  Overflow rounds to +-inf as IEEE does.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

// Element-type tags.  Every kernel moves data in 16-byte chunks: 8 elements of a
// 16-bit type or 4 fp32 elements.
struct TBF16 {
  static constexpr int kBytes = 2;
  static constexpr int kPerChunk = 8;
  static constexpr gns_dtype kId = GNS_BF16;
  __device__ static float to_f32(uint32_t bits) { return bf16_bits_to_f32(bits); }
  __device__ static uint32_t from_f32(float v) { return f32_to_bf16_bits(v); }
};
struct TF16 {
  static constexpr int kBytes = 2;
  static constexpr int kPerChunk = 8;
  static constexpr gns_dtype kId = GNS_F16;
  __device__ static float to_f32(uint32_t bits) { return f16_bits_to_f32(bits); }
  __device__ static uint32_t from_f32(float v) { return f32_to_f16_bits(v); }
};
struct TF32 {
  static constexpr int kBytes = 4;
  static constexpr int kPerChunk = 4;
  static constexpr gns_dtype kId = GNS_F32;
  __device__ static float to_f32(uint32_t bits) { return __uint_as_float(bits); }
  __device__ static uint32_t from_f32(float v) { return __float_as_uint(v); }
};

// Element i of a 16-byte chunk, widened to fp32.
template <class T>
__device__ __forceinline__ float chunk_elem(const uint4& c, int i) {
  const uint32_t* w = reinterpret_cast<const uint32_t*>(&c);
  if constexpr (T::kBytes == 4) {
    return __uint_as_float(w[i]);
  } else {
    uint32_t word = w[i >> 1];
    return T::to_f32((i & 1) ? (word >> 16) : (word & 0xffffu));
  }
}

// One MFMA k-step on a 16x16 output fragment.  `a` and `b` each hold one 16-byte
// chunk per lane: lane l carries row/col (l % 16) and k-group (l / 16).  For 16-bit
// types one v_mfma_f32_16x16x32 consumes all 8 values (k = 8*group + j); for fp32,
// four v_mfma_f32_16x16x4 consume element j of each lane in step j, so step j covers
// k = 4*group + j.  Any fixed k permutation is fine as long as A and B share it.
// The call passes (b, a): the accumulator then holds the fragment transposed, i.e.
// lane l owns row (l % 16) of the output and 4 consecutive columns 4*(l/16)+i.
template <class T>
__device__ __forceinline__ void mfma_step(f32x4_t& acc, const uint4& a, const uint4& b) {
  if constexpr (T::kId == GNS_BF16) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, b),
                                                 __builtin_bit_cast(bf16x8_t, a), acc, 0, 0, 0);
  } else if constexpr (T::kId == GNS_F16) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, b),
                                                __builtin_bit_cast(f16x8_t, a), acc, 0, 0, 0);
  } else {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(b.x), __uint_as_float(a.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(b.y), __uint_as_float(a.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(b.z), __uint_as_float(a.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(b.w), __uint_as_float(a.w), acc, 0, 0, 0);
  }
}

// LDS tile rows are 128 bytes = 8 chunks.  gfx950's LDS serves 256 bytes per clock
// (64 banks) to ds_read_b128, i.e. 16 lanes at a time; an MFMA fragment read has 16
// lanes on 16 consecutive rows at the same logical chunk.  With the physical chunk
// c ^ ((r >> 1) & 7), rows 2j and 2j+1 (one 256-byte bank window) sit at slot c ^ j
// of their two halves, so the 16 rows hit 16 distinct 16-byte slots: conflict-free.
// (Measured on MI355X: 202 B/clk/CU for this read pattern, the same as a linear
// read; the variant c ^ (r & 7) ^ ((r >> 3) & 1) reached only 114 B/clk.)  Row-wise
// writes (8 lanes per 128-byte row) stay conflict-free under any such permutation.
__device__ __forceinline__ int swz(int row, int chunk) {
  return chunk ^ ((row >> 1) & 7);
}

// Raw buffer resource over [base, base + bytes): loads at offsets past the end
// return zero in hardware, which gives branch-free predication of tile edges.
constexpr uint32_t kOutOfRange = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t offset) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)offset, 0, 0));
}

// hipGetLastError() reports the last error of ANY runtime call on this thread (for
// example hipErrorNotReady left by an event query of the caller).  Launchers clear
// it right before a launch so the check after the launch sees only that launch.
inline void clear_stale_error() { (void)hipGetLastError(); }

// 64-bit flat index helper.
__device__ __forceinline__ long long idx2(long long r, long long ld, long long c) { return r * ld + c; }

}  // namespace gns
