// BF16 -> FP8-E4M3FN write path for gfx950: quantise freshly computed KV rows
// and scatter them into their pool slots, the CastToFP8 step of
// "When a Faster Kernel Doesn't Speed Up Serving" (Step 3: set_kv_buffer
// copies the new BF16 KV into the FP8 cache).
//
// Pure bandwidth work: 2 bytes read and 1 byte written per element, plus one
// 4-byte slot id per row.  A row of 576 elements is handled by 72 lanes, each
// with one 16-byte load (8 BF16 values) and one 8-byte store (8 codes), so the
// lanes of a row read and write it contiguously.
//
// Encoding: gfx950's v_cvt_pk_fp8_f32 rounds a float32 to the nearest
// E4M3FN value, ties to the even code, gives subnormal codes below 2^-6, and
// gives NaN for magnitudes above 464 (the midpoint between 448 and the next
// step up) and for infinities -- the float -> Float8_e4m3fn copy rule -- for
// every non-NaN input; for a NaN input it returns 0xFF whatever the sign.  So
// the kernel converts magnitudes, |x| * inv_scale (the absolute value is a
// free source modifier of the multiply), which gives codes 0x00..0x7E or 0x7F
// for overflow, 0xFF for NaN, keeps the low 7 bits, and inserts each source
// sign bit as bit 7: NaN then gives 0x7F or 0xFF by its sign.  About 3 VALU
// operations per element, so the kernel stays bound by memory.
#include "device_common.h"
#include "launch.h"

namespace fp8mla {
namespace {

constexpr uint32_t kF32Bits448 = 0x43E00000u;     // largest finite E4M3FN value
constexpr uint32_t kF32BitsInf = 0x7F800000u;

// |x| * inv_scale for the BF16 value whose bits are the high half of `b32`
// (low half zero); with SATURATE the magnitude is clamped to 448 unless it
// is NaN (compared as bit patterns, which order like the values for
// non-negative floats).
template <bool SATURATE>
__device__ __forceinline__ float scaled_magnitude(uint32_t b32, float inv_scale) {
  const float y = fabsf(__builtin_bit_cast(float, b32)) * inv_scale;
  if constexpr (SATURATE) {
    const uint32_t a = __builtin_bit_cast(uint32_t, y);
    return __builtin_bit_cast(float, a > kF32BitsInf ? a : min(a, kF32Bits448));
  } else {
    return y;
  }
}

// Four BF16 values (two 32-bit words, element j in bits 16j..16j+15 of the
// pair) -> four E4M3FN codes, byte j = element j.
template <bool SATURATE>
__device__ __forceinline__ uint32_t encode4(uint32_t w0, uint32_t w1, float inv_scale) {
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(scaled_magnitude<SATURATE>(w0 << 16, inv_scale),
                                          scaled_magnitude<SATURATE>(w0 & 0xFFFF0000u, inv_scale),
                                          0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(scaled_magnitude<SATURATE>(w1 << 16, inv_scale),
                                      scaled_magnitude<SATURATE>(w1 & 0xFFFF0000u, inv_scale),
                                      r, true);
  // the high byte of each BF16 value holds its sign in bit 7: bytes 1, 3 of
  // w0 and bytes 1, 3 of w1 (indices 1, 3, 5, 7 of the pair w1:w0)
  const uint32_t hi_bytes = __builtin_amdgcn_perm(w1, w0, 0x07050301u);
  return ((uint32_t)r & 0x7F7F7F7Fu) | (hi_bytes & 0x80808080u);
}

// Eight BF16 values (16 bytes) -> eight codes (8 bytes).
template <bool SATURATE>
__device__ __forceinline__ u32x2_t encode8(const u32x4_t w, float inv_scale) {
  u32x2_t o;
  o[0] = encode4<SATURATE>(w[0], w[1], inv_scale);
  o[1] = encode4<SATURATE>(w[2], w[3], inv_scale);
  return o;
}

// One block of 576 lanes covers 8 rows per pass (72 lanes x 8 elements per
// row) and SC_UNROLL passes, i.e. 32 consecutive source rows; every lane keeps
// SC_UNROLL loads in flight.  Rows whose slot is outside [0, num_slots) are
// read but not written.
constexpr int SC_LANES_PER_ROW = KV_WIDTH / 8;                      // 72
constexpr int SC_ROWS_PER_PASS = 8;
constexpr int SC_THREADS = SC_ROWS_PER_PASS * SC_LANES_PER_ROW;     // 576 = 9 waves
constexpr int SC_UNROLL = 4;
constexpr int SC_ROWS_PER_BLOCK = SC_ROWS_PER_PASS * SC_UNROLL;     // 32

template <bool SATURATE>
__global__ __launch_bounds__(SC_THREADS) void scatter_cast_kernel(
    const uint16_t* __restrict__ src, int64_t src_row_stride, int64_t n,
    const int32_t* __restrict__ slots, uint8_t* __restrict__ pool, uint32_t num_slots,
    float inv_scale) {
  const int rr = threadIdx.x / SC_LANES_PER_ROW;
  const int c = threadIdx.x - rr * SC_LANES_PER_ROW;
  const int64_t r0 = (int64_t)blockIdx.x * SC_ROWS_PER_BLOCK + rr;
  uint32_t slot[SC_UNROLL];
#pragma unroll
  for (int u = 0; u < SC_UNROLL; ++u) {
    const int64_t r = r0 + u * SC_ROWS_PER_PASS;
    slot[u] = r < n ? (uint32_t)slots[r] : num_slots;  // negative ids wrap past num_slots
  }
  u32x4_t v[SC_UNROLL];
#pragma unroll
  for (int u = 0; u < SC_UNROLL; ++u) {
    const int64_t r = r0 + u * SC_ROWS_PER_PASS;
    if (r < n) v[u] = load16_nt(src + r * src_row_stride + 8 * c);
  }
#pragma unroll
  for (int u = 0; u < SC_UNROLL; ++u) {
    const int64_t r = r0 + u * SC_ROWS_PER_PASS;
    if (r < n && slot[u] < num_slots)
      store8_dev(pool + (uint64_t)slot[u] * KV_WIDTH + 8 * c, encode8<SATURATE>(v[u], inv_scale));
  }
}

}  // namespace

hipError_t launch_scatter_cast(const uint16_t* src, int64_t src_row_stride, int64_t n,
                               const int32_t* slots, uint8_t* pool, int64_t num_slots,
                               float inv_scale, bool saturate, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int64_t blocks = (n + SC_ROWS_PER_BLOCK - 1) / SC_ROWS_PER_BLOCK;
  if (saturate)
    hipLaunchKernelGGL(scatter_cast_kernel<true>, dim3((unsigned)blocks), dim3(SC_THREADS), 0,
                       stream, src, src_row_stride, n, slots, pool, (uint32_t)num_slots, inv_scale);
  else
    hipLaunchKernelGGL(scatter_cast_kernel<false>, dim3((unsigned)blocks), dim3(SC_THREADS), 0,
                       stream, src, src_row_stride, n, slots, pool, (uint32_t)num_slots, inv_scale);
  return hipGetLastError();
}

}  // namespace fp8mla
