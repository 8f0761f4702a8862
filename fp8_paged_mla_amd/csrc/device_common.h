// Device-side helpers shared by the gfx950 kernels of libfp8mla.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8mla {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(2))) int i32x2_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

constexpr int KV_WIDTH = 576;  // bytes per latent row: 512 latent + 64 rope
constexpr int V_WIDTH = 512;   // value operand = first 512 columns
constexpr int KV_CHUNKS = KV_WIDTH / 16;  // 36 chunks of 16 bytes per row

// Two E4M3FN bytes (bytes 0-1 of w when HI is false, bytes 2-3 when true)
// to two BF16 values packed low-to-high.  gfx950's scaled converter with a
// unit scale is exact for every finite E4M3FN code (each is a BF16 value);
// it returns 0xFFC0 for both NaN codes.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
  bf16x2_t r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
  return __builtin_bit_cast(uint32_t, r);
}

// Eight E4M3FN bytes (lo = bytes 0-3, hi = bytes 4-7) to an MFMA bf16x8 operand,
// element j = byte j.
__device__ __forceinline__ bf16x8_t e4m3x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  u32x4_t v;
  v[0] = e4m3x2_to_bf16x2<false>(lo);
  v[1] = e4m3x2_to_bf16x2<true>(lo);
  v[2] = e4m3x2_to_bf16x2<false>(hi);
  v[3] = e4m3x2_to_bf16x2<true>(hi);
  return __builtin_bit_cast(bf16x8_t, v);
}

// The same for FP16: every finite E4M3FN value (at most 448 in magnitude,
// at least 2^-9 when not zero) is also an FP16 value, so this is exact too.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_f16x2(uint32_t w) {
  f16x2_t r = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI);
  return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ f16x8_t e4m3x8_to_f16x8(uint32_t lo, uint32_t hi) {
  u32x4_t v;
  v[0] = e4m3x2_to_f16x2<false>(lo);
  v[1] = e4m3x2_to_f16x2<true>(lo);
  v[2] = e4m3x2_to_f16x2<false>(hi);
  v[3] = e4m3x2_to_f16x2<true>(hi);
  return __builtin_bit_cast(f16x8_t, v);
}

// Streaming 16-byte accesses (non-temporal: data used once, keep it out of
// the way of cached data).
__device__ __forceinline__ u32x4_t load16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}
__device__ __forceinline__ u32x2_t load8_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
}
__device__ __forceinline__ void store16_nt(void* p, u32x4_t v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p));
}
// 16-byte store at device scope (sc1): written through to the device's
// coherence point instead of being kept in the XCD's L2.  The gather-cast's
// 18 KB row-block writes run 11% faster this way on MI355X, the full-pool
// cast's streaming writes 8% slower (they keep store16_nt).
__device__ __forceinline__ void store16_dev(void* p, u32x4_t v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1" ::"v"(p), "v"(v) : "memory");
}
// 8-byte store at device scope; the write path's scattered 576-byte rows
// measured 2% faster this way than with the default policy (non-temporal
// stores: 13% slower).
__device__ __forceinline__ void store8_dev(void* p, u32x2_t v) {
  asm volatile("global_store_dwordx2 %0, %1, off sc1" ::"v"(p), "v"(v) : "memory");
}

// Per byte of w: 0x80 where the byte is an E4M3FN NaN (low 7 bits all ones).
__device__ __forceinline__ uint32_t e4m3_nan_flags(uint32_t w) {
  return ((w & 0x7F7F7F7Fu) + 0x01010101u) & 0x80808080u;
}

// Round-to-nearest-even float -> BF16 bits (gfx950 converts in hardware).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __builtin_bit_cast(float, bits16 << 16);
}

}  // namespace fp8mla
