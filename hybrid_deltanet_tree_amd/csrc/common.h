// common.h - device helpers shared by the kernel sources of libhdt (gfx950).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <type_traits>

#include "launch.h"

namespace hdt {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <bool BF>
using io_t = typename std::conditional<BF, uint16_t, float>::type;

// Element i of an io-dtype array (bf16 bits or float32), widened to float.
template <bool BF>
__device__ __forceinline__ float ld_io(const void *p, int64_t i) {
  if constexpr (BF) {
    return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t *>(p)[i]) << 16);
  } else {
    return static_cast<const float *>(p)[i];
  }
}

// Round to bf16, nearest even.
__device__ __forceinline__ uint16_t bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

template <bool BF>
__device__ __forceinline__ void st_io(void *p, int64_t i, float v) {
  if constexpr (BF) {
    static_cast<uint16_t *>(p)[i] = bf16_bits(v);
  } else {
    static_cast<float *>(p)[i] = v;
  }
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Workgroup barrier that waits only for this wave's LDS operations: vector-memory
// loads still in flight stay in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt not waited
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Workgroup barrier without a memory fence: the compiler may not move memory
// accesses across it, and the hardware does not wait for outstanding operations.
__device__ __forceinline__ void bare_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Wait until at most N of this wave's vector-memory operations are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N < 64, "vmcnt has 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Buffer resource over `bytes` bytes from `base`: loads at or past the end read
// zeros and move no data.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}

// Brings the 64-byte lines of a uniform (kernel-argument) region into the scalar
// cache with loads issued together and one wait, so that later reads of its fields
// hit that cache instead of each paying a memory round trip in turn.  `bytes` is at
// most 384; `tail` is one more uniform address (the launch's shared fields).
__device__ __forceinline__ void scalar_touch(const void *base, int bytes, const void *tail) {
  const unsigned char *b = static_cast<const unsigned char *>(base);
  const int last = bytes - 4;
  uint32_t x[6];
#pragma unroll
  for (int i = 0; i < 6; ++i) x[i] = *reinterpret_cast<const uint32_t *>(b + min(64 * i, last));
  const uint32_t y = *static_cast<const uint32_t *>(tail);
  asm volatile("" ::"s"(x[0]), "s"(x[1]), "s"(x[2]), "s"(x[3]), "s"(x[4]), "s"(x[5]), "s"(y));
}

// LDS byte address of a pointer into shared memory, and back.
typedef __attribute__((address_space(3))) unsigned char lds_u8;
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_u8 *)(p)));
}
__device__ __forceinline__ const lds_u8 *lds_ptr(uint32_t a) {
  return reinterpret_cast<const lds_u8 *>(static_cast<uintptr_t>(a));
}
__device__ __forceinline__ shortx4 ds_read_tr_at(uint32_t a) {
  typedef __attribute__((address_space(3))) shortx4 *lds_v4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4)(lds_ptr(a)));
}

// Transposed LDS read (ds_read_b64_tr_b16).  In each group of 16 lanes, lane p
// supplies the address of 4 consecutive bf16 values; lane j receives element j % 4
// of the values addressed by lanes 4e + j / 4, for e = 0..3.
__device__ __forceinline__ shortx4 ds_read_tr(const unsigned char *p) {
  typedef __attribute__((address_space(3))) shortx4 *lds_v4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_v4)((__attribute__((address_space(3))) unsigned char *)(p)));
}

// Max and sum over the lanes l, l ^ 16, l ^ 32, l ^ 48 (the four 16-lane rows).
// Both halves of each swap add or compare the same two values, so every lane
// gets the same bits.
__device__ __forceinline__ float rows4_max(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float rows4_sum(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Max and sum over the lanes l and l ^ 32 (the two halves of a wave).  Both halves
// of the swap combine the same two values, so both lanes get the same bits.
__device__ __forceinline__ float pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace hdt
