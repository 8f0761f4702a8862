// FP8-E4M3FN -> BF16 cast kernels for gfx950: the full-pool cast and the
// gather-then-cast fallback.
//
// Both are pure bandwidth work (1 byte read, 2 bytes written per element, plus
// 4 index bytes per gathered row), so they are written for coalescing, not
// for arithmetic: 8-byte loads and 16-byte stores per lane that make every
// wave instruction one contiguous span, several loads in flight per lane, and
// one conversion instruction per two elements.
#include "device_common.h"
#include "launch.h"

namespace fp8mla {
namespace {

// BF16 pair with each 0xFFC0 half (the converter's NaN) replaced by 0x7FC0.
__device__ __forceinline__ uint32_t canonical_nan(uint32_t x) {
  if ((x & 0xFFFFu) == 0xFFC0u) x = (x & 0xFFFF0000u) | 0x7FC0u;
  if ((x >> 16) == 0xFFC0u) x = (x & 0x0000FFFFu) | 0x7FC00000u;
  return x;
}

// Eight E4M3FN bytes -> eight BF16 values (16 bytes).  The hardware
// converter gives 0xFFC0 for a NaN code; the torch .to() cast the pages use
// gives the canonical 0x7FC0, so NaN lanes are rewritten (a rare branch,
// tested with 3 integer ops per 4 bytes).
__device__ __forceinline__ u32x4_t convert8(const u32x2_t in) {
  u32x4_t o;
  o[0] = e4m3x2_to_bf16x2<false>(in[0]);
  o[1] = e4m3x2_to_bf16x2<true>(in[0]);
  o[2] = e4m3x2_to_bf16x2<false>(in[1]);
  o[3] = e4m3x2_to_bf16x2<true>(in[1]);
  if (__builtin_expect((e4m3_nan_flags(in[0]) | e4m3_nan_flags(in[1])) != 0u, 0)) {
    o[0] = canonical_nan(o[0]);
    o[1] = canonical_nan(o[1]);
    o[2] = canonical_nan(o[2]);
    o[3] = canonical_nan(o[3]);
  }
  return o;
}

constexpr int CAST_THREADS = 256;
constexpr int CAST_UNROLL = 8;
constexpr int CAST_BLOCKS_PER_CU = 32;

// Grid-stride over 8-byte input chunks: lane i reads bytes 8i..8i+7 and
// writes output bytes 16i..16i+15, so every load and store instruction of a
// wave covers one contiguous span (512 B in, 1 KB out).  Stores that leave
// half-written lines behind (two 16-byte stores per lane at a 32-byte
// stride) cost about a quarter more HBM write traffic on this part.  Each
// lane keeps CAST_UNROLL loads in flight; accesses are non-temporal since
// pool and copy are streamed once.
__global__ __launch_bounds__(CAST_THREADS) void cast_pool_kernel(const u32x2_t* __restrict__ in,
                                                                 u32x4_t* __restrict__ out,
                                                                 int64_t n8) {
  const int64_t stride = (int64_t)gridDim.x * CAST_THREADS;
  int64_t i = (int64_t)blockIdx.x * CAST_THREADS + threadIdx.x;
  for (; i + (CAST_UNROLL - 1) * stride < n8; i += CAST_UNROLL * stride) {
    u32x2_t v[CAST_UNROLL];
#pragma unroll
    for (int u = 0; u < CAST_UNROLL; ++u) v[u] = load8_nt(&in[i + u * stride]);
#pragma unroll
    for (int u = 0; u < CAST_UNROLL; ++u) store16_nt(&out[i + u * stride], convert8(v[u]));
  }
  for (; i < n8; i += stride) store16_nt(&out[i], convert8(load8_nt(&in[i])));
}

// Gather-then-cast: one block of 576 lanes covers 8 rows per pass (72 lanes
// x 8 bytes per row) and GATHER_UNROLL passes, i.e. 64 consecutive output
// rows.  Lanes of a row read its 576 contiguous bytes; the block's output
// rows are contiguous, 16 bytes per lane.
constexpr int GATHER_LANES_PER_ROW = KV_WIDTH / 8;                       // 72
constexpr int GATHER_ROWS_PER_PASS = 8;
constexpr int GATHER_THREADS = GATHER_ROWS_PER_PASS * GATHER_LANES_PER_ROW;  // 576 = 9 waves
constexpr int GATHER_UNROLL = 8;
constexpr int GATHER_ROWS_PER_BLOCK = GATHER_ROWS_PER_PASS * GATHER_UNROLL;  // 64

__global__ __launch_bounds__(GATHER_THREADS) void gather_cast_kernel(
    const uint8_t* __restrict__ pool, uint32_t max_slot, const int32_t* __restrict__ indices,
    int64_t n, u32x4_t* __restrict__ out) {
  const int rr = threadIdx.x / GATHER_LANES_PER_ROW;
  const int c = threadIdx.x - rr * GATHER_LANES_PER_ROW;
  const int64_t r0 = (int64_t)blockIdx.x * GATHER_ROWS_PER_BLOCK + rr;
  uint32_t slot[GATHER_UNROLL];
#pragma unroll
  for (int u = 0; u < GATHER_UNROLL; ++u) {
    const int64_t r = r0 + u * GATHER_ROWS_PER_PASS;
    const uint32_t s = r < n ? (uint32_t)indices[r] : 0u;
    slot[u] = s < max_slot ? s : max_slot;  // negative or too large -> last slot
  }
  u32x2_t v[GATHER_UNROLL];
#pragma unroll
  for (int u = 0; u < GATHER_UNROLL; ++u) {
    const int64_t r = r0 + u * GATHER_ROWS_PER_PASS;
    if (r < n) v[u] = load8_nt(pool + (uint64_t)slot[u] * KV_WIDTH + 8 * c);
  }
#pragma unroll
  for (int u = 0; u < GATHER_UNROLL; ++u) {
    const int64_t r = r0 + u * GATHER_ROWS_PER_PASS;
    if (r < n) store16_nt(&out[r * GATHER_LANES_PER_ROW + c], convert8(v[u]));
  }
}

}  // namespace

hipError_t launch_cast_pool(const uint8_t* pool, int64_t num_slots, uint16_t* out,
                            hipStream_t stream, int num_cus) {
  const int64_t n8 = num_slots * (KV_WIDTH / 8);
  if (n8 == 0) return hipSuccess;
  int64_t blocks = (n8 + CAST_THREADS - 1) / CAST_THREADS;
  const int64_t cap = (int64_t)num_cus * CAST_BLOCKS_PER_CU;
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL(cast_pool_kernel, dim3((unsigned)blocks), dim3(CAST_THREADS), 0, stream,
                     reinterpret_cast<const u32x2_t*>(pool), reinterpret_cast<u32x4_t*>(out), n8);
  return hipGetLastError();
}

hipError_t launch_gather_cast(const uint8_t* pool, int64_t num_slots, const int32_t* indices,
                              int64_t n, uint16_t* out, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int64_t blocks = (n + GATHER_ROWS_PER_BLOCK - 1) / GATHER_ROWS_PER_BLOCK;
  hipLaunchKernelGGL(gather_cast_kernel, dim3((unsigned)blocks), dim3(GATHER_THREADS), 0, stream,
                     pool, (uint32_t)(num_slots - 1), indices, n, reinterpret_cast<u32x4_t*>(out));
  return hipGetLastError();
}

}  // namespace fp8mla
