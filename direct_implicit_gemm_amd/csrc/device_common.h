// device_common.h -- device-side helpers shared by the libconv kernels:
// storage-dtype conversions and bounds-checked buffer access.
//
// Every global load and store in libconv goes through a buffer resource whose
// size is the tensor's byte size: an access outside the tensor reads zero and
// a store outside it is dropped by the hardware, so an indexing mistake can
// produce a wrong value but never a memory fault.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace libconv {

enum : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

// Word 3 of a gfx9-family buffer descriptor (raw, untyped 32-bit access).
constexpr int kBufferWord3 = 0x00020000;

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, kBufferWord3);
}

// Byte offset that reads as zero from any buffer made by make_rsrc (tensors
// are below 2^31 bytes; offsets are unsigned 32-bit).
constexpr int kOobOffset = -16;

// An offset past the end of every tensor (all are below 0x7fff0000 bytes)
// that stays past the end when a scalar offset below 2^31 is added to it
// (the range check covers the sum, and it must not wrap around 2^32).
constexpr int kFarOffset = 0x7ffff000;

// `ok ? off : kOobOffset`, computed in a register the optimiser treats as
// opaque.  Written as a plain select, the compiler may turn
// load(select(c, a, b)) into two loads on two branches, and the join after
// them makes the wave wait for every load before the next one issues.
__device__ __forceinline__ int guard_offset(bool ok, int off) {
  int v = ok ? off : kOobOffset;
  asm("" : "+v"(v));
  return v;
}

// Cache policy of the stores that write a call's output (the aux operand of
// the buffer store builtins): non-temporal, so that output lines stream out
// to memory while the kernel runs instead of sitting dirty in L2 until the
// write-back at its end, and push fewer of the lines that later workgroups
// read out of L2.  Split-K partial sums and packed weights, which the next
// kernel reads back at once, keep the default policy.
constexpr int kOutPolicy = 2;

// --- storage element <-> fp32 -------------------------------------------
template <int DT> struct Elem;

template <> struct Elem<DT_F32> {
  static constexpr int bytes = 4;
  __device__ static __forceinline__ float load(__amdgpu_buffer_rsrc_t r, int byte_off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0));
  }
  __device__ static __forceinline__ void store(float v, __amdgpu_buffer_rsrc_t r, int byte_off) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, byte_off, 0, 0);
  }
  __device__ static __forceinline__ void store_out(float v, __amdgpu_buffer_rsrc_t r, int byte_off) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, byte_off, 0,
                                          kOutPolicy);
  }
  __device__ static __forceinline__ uint32_t load_bits(__amdgpu_buffer_rsrc_t r, int byte_off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0);
  }
  __device__ static __forceinline__ float bits_to_f32(uint32_t b) { return __builtin_bit_cast(float, b); }
  // the element exactly as loaded, in its own width
  using raw_t = uint32_t;
  __device__ static __forceinline__ raw_t load_raw(__amdgpu_buffer_rsrc_t r, int byte_off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0);
  }
};

template <> struct Elem<DT_F16> {
  static constexpr int bytes = 2;
  using raw_t = uint16_t;
  __device__ static __forceinline__ raw_t load_raw(__amdgpu_buffer_rsrc_t r, int byte_off) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, byte_off, 0, 0);
  }
  __device__ static __forceinline__ float bits_to_f32(uint32_t b) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
  }
  __device__ static __forceinline__ uint32_t load_bits(__amdgpu_buffer_rsrc_t r, int byte_off) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, byte_off, 0, 0);
  }
  __device__ static __forceinline__ float load(__amdgpu_buffer_rsrc_t r, int byte_off) {
    return bits_to_f32(load_bits(r, byte_off));
  }
  // Round to nearest even (the default rounding mode of the conversion).
  __device__ static __forceinline__ uint16_t from_f32(float v) {
    return __builtin_bit_cast(uint16_t, (_Float16)v);
  }
  __device__ static __forceinline__ void store(float v, __amdgpu_buffer_rsrc_t r, int byte_off) {
    __builtin_amdgcn_raw_buffer_store_b16(from_f32(v), r, byte_off, 0, 0);
  }
  __device__ static __forceinline__ void store_out(float v, __amdgpu_buffer_rsrc_t r, int byte_off) {
    __builtin_amdgcn_raw_buffer_store_b16(from_f32(v), r, byte_off, 0, kOutPolicy);
  }
};

template <> struct Elem<DT_BF16> {
  static constexpr int bytes = 2;
  using raw_t = uint16_t;
  __device__ static __forceinline__ raw_t load_raw(__amdgpu_buffer_rsrc_t r, int byte_off) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, byte_off, 0, 0);
  }
  __device__ static __forceinline__ float bits_to_f32(uint32_t b) {
    return __builtin_bit_cast(float, (uint32_t)(b & 0xffffu) << 16);
  }
  __device__ static __forceinline__ uint32_t load_bits(__amdgpu_buffer_rsrc_t r, int byte_off) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, byte_off, 0, 0);
  }
  __device__ static __forceinline__ float load(__amdgpu_buffer_rsrc_t r, int byte_off) {
    return bits_to_f32(load_bits(r, byte_off));
  }
  // Round to nearest even.
  __device__ static __forceinline__ uint16_t from_f32(float v) {
    return __builtin_bit_cast(uint16_t, (__bf16)v);
  }
  __device__ static __forceinline__ void store(float v, __amdgpu_buffer_rsrc_t r, int byte_off) {
    __builtin_amdgcn_raw_buffer_store_b16(from_f32(v), r, byte_off, 0, 0);
  }
  __device__ static __forceinline__ void store_out(float v, __amdgpu_buffer_rsrc_t r, int byte_off) {
    __builtin_amdgcn_raw_buffer_store_b16(from_f32(v), r, byte_off, 0, kOutPolicy);
  }
};

// Bias + activation, applied to the fp32 accumulator before the one rounding
// to the storage dtype.  ReLU maps NaN to 0, like max(v, 0) on the host.
__device__ __forceinline__ float epilogue(float acc, float bias, int relu) {
  float v = acc + bias;
  if (relu) v = (v > 0.0f) ? v : 0.0f;
  return v;
}

}  // namespace libconv
