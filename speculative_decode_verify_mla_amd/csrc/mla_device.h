// Device helpers shared by the gfx950 kernels of libmla_verify (HIP device
// code only; not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mlav {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

#define LDS_AS __attribute__((address_space(3)))

constexpr unsigned kBufferConfig = 0x00020000u;  // raw buffer, 32-bit data format (gfx9 family)

// Generic -> LDS address-space pointers (the arrays live in LDS; the casts only
// let the compiler emit ds_* / LDS-DMA instructions directly).
__device__ __forceinline__ bf16x8 lds_read16(const uint8_t* base, unsigned off) {
  const LDS_AS uint8_t* p = (const LDS_AS uint8_t*)(base) + off;
  return *(const LDS_AS bf16x8*)p;
}

// Transposing read (ds_read_b64_tr_b16). The intrinsic carries no type-based
// alias information, and an LDS read without any is made to wait for every
// buffer->LDS DMA in flight (s_waitcnt vmcnt(0)), the next tile's loads included.
// The restrict qualifier attaches alias scopes, which lifts that wait, as for
// the plain typed reads. Callers order DMA writes before reads themselves
// (s_waitcnt on the loads, then a barrier when other waves issued them).
__device__ __forceinline__ bf16x4 lds_read_tr(const uint8_t* __restrict__ base, unsigned off) {
  LDS_AS uint8_t* p = (LDS_AS uint8_t*)(base) + off;
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)p);
}

// 16 bytes per lane from a buffer straight into LDS. kNonTemporal sets the
// load's nt cache-policy bit (rows that no other workgroup will read).
template <bool kNonTemporal = false>
__device__ __forceinline__ void buffer_to_lds(__amdgpu_buffer_rsrc_t rsrc, uint8_t* lds_dst,
                                              unsigned voffset) {
  constexpr int kPolicy = kNonTemporal ? 2 : 0;  // gfx950 cache-policy bits: nt = 2
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (LDS_AS void*)(lds_dst), 16, voffset, 0, 0, kPolicy);
}

// 8 bytes per lane stored through a buffer descriptor with the sc0 and sc1
// cache-policy bits set (system scope: written through the caches rather than
// left dirty in L2 at the kernel's end).
__device__ __forceinline__ void buffer_store_b64_wt(u32x2 v, __amdgpu_buffer_rsrc_t rsrc, unsigned voffset) {
  constexpr int kPolicy = 1 | 16;  // gfx950 cache-policy bits: sc0 = 1, sc1 = 16
  __builtin_amdgcn_raw_buffer_store_b64(v, rsrc, (int)voffset, 0, kPolicy);
}

// Buffer descriptors are wave-uniform; readfirstlane keeps them in SGPRs even
// when the compiler cannot prove uniformity (it would otherwise emit a loop).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t v = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  void* ub = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes),
                                           (int)kBufferConfig);
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Two floats -> two packed bf16 (low = a) in one conversion, round to nearest
// even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

}  // namespace mlav
