// FP8-E4M3FN -> BF16 cast kernels for gfx950: the full-pool cast and the
// gather-then-cast fallback.
//
// Both are pure bandwidth work (1 byte read, 2 bytes written per element, plus
// 4 index bytes per gathered row), so they are written for coalescing, not
// for arithmetic: 16-byte loads, 32-byte stores per lane, several loads in
// flight per lane, and one conversion instruction per two elements.
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

// Sixteen E4M3FN bytes -> sixteen BF16 values (32 bytes).  The hardware
// converter gives 0xFFC0 for a NaN code; the torch .to() cast the pages use
// gives the canonical 0x7FC0, so NaN lanes are rewritten (rare, checked with
// a 3-op test per 4 bytes).
__device__ __forceinline__ void convert16(const u32x4_t in, u32x4_t& o0, u32x4_t& o1) {
  o0[0] = e4m3x2_to_bf16x2<false>(in[0]);
  o0[1] = e4m3x2_to_bf16x2<true>(in[0]);
  o0[2] = e4m3x2_to_bf16x2<false>(in[1]);
  o0[3] = e4m3x2_to_bf16x2<true>(in[1]);
  o1[0] = e4m3x2_to_bf16x2<false>(in[2]);
  o1[1] = e4m3x2_to_bf16x2<true>(in[2]);
  o1[2] = e4m3x2_to_bf16x2<false>(in[3]);
  o1[3] = e4m3x2_to_bf16x2<true>(in[3]);
  const uint32_t nan = e4m3_nan_flags(in[0]) | e4m3_nan_flags(in[1]) |
                       e4m3_nan_flags(in[2]) | e4m3_nan_flags(in[3]);
  if (__builtin_expect(nan != 0u, 0)) {
    o0[0] = canonical_nan(o0[0]);
    o0[1] = canonical_nan(o0[1]);
    o0[2] = canonical_nan(o0[2]);
    o0[3] = canonical_nan(o0[3]);
    o1[0] = canonical_nan(o1[0]);
    o1[1] = canonical_nan(o1[1]);
    o1[2] = canonical_nan(o1[2]);
    o1[3] = canonical_nan(o1[3]);
  }
}

constexpr int CAST_THREADS = 256;
constexpr int CAST_UNROLL = 4;

// Grid-stride over 16-byte input chunks; each lane keeps CAST_UNROLL loads
// in flight.  Input and output are streamed once: non-temporal accesses keep
// them from evicting other data from the caches.
__global__ __launch_bounds__(CAST_THREADS) void cast_pool_kernel(const u32x4_t* __restrict__ in,
                                                                 u32x4_t* __restrict__ out,
                                                                 int64_t nchunks) {
  const int64_t stride = (int64_t)gridDim.x * CAST_THREADS;
  int64_t i = (int64_t)blockIdx.x * CAST_THREADS + threadIdx.x;
  for (; i + (CAST_UNROLL - 1) * stride < nchunks; i += CAST_UNROLL * stride) {
    u32x4_t v[CAST_UNROLL];
#pragma unroll
    for (int u = 0; u < CAST_UNROLL; ++u) v[u] = load16_nt(&in[i + u * stride]);
#pragma unroll
    for (int u = 0; u < CAST_UNROLL; ++u) {
      u32x4_t o0, o1;
      convert16(v[u], o0, o1);
      const int64_t j = 2 * (i + u * stride);
      store16_nt(&out[j], o0);
      store16_nt(&out[j + 1], o1);
    }
  }
  for (; i < nchunks; i += stride) {
    u32x4_t o0, o1;
    convert16(load16_nt(&in[i]), o0, o1);
    store16_nt(&out[2 * i], o0);
    store16_nt(&out[2 * i + 1], o1);
  }
}

// One block = 64 output rows; 576 lanes = 16 rows x 36 chunks, each lane
// handling its chunk of rows rr, rr+16, rr+32, rr+48.  Lanes of a row read
// its 576 contiguous bytes; consecutive lanes write consecutive 32 bytes.
constexpr int GATHER_ROWS_PER_PASS = 16;
constexpr int GATHER_THREADS = GATHER_ROWS_PER_PASS * KV_CHUNKS;  // 576 = 9 waves
constexpr int GATHER_UNROLL = 4;
constexpr int GATHER_ROWS_PER_BLOCK = GATHER_ROWS_PER_PASS * GATHER_UNROLL;

__global__ __launch_bounds__(GATHER_THREADS) void gather_cast_kernel(
    const uint8_t* __restrict__ pool, uint32_t max_slot, const int32_t* __restrict__ indices,
    int64_t n, u32x4_t* __restrict__ out) {
  const int rr = threadIdx.x / KV_CHUNKS;
  const int c = threadIdx.x - rr * KV_CHUNKS;
  const int64_t r0 = (int64_t)blockIdx.x * GATHER_ROWS_PER_BLOCK + rr;
  uint32_t slot[GATHER_UNROLL];
#pragma unroll
  for (int u = 0; u < GATHER_UNROLL; ++u) {
    const int64_t r = r0 + u * GATHER_ROWS_PER_PASS;
    const uint32_t s = r < n ? (uint32_t)indices[r] : 0u;
    slot[u] = s < max_slot ? s : max_slot;  // negative or too large -> last slot
  }
  u32x4_t v[GATHER_UNROLL];
#pragma unroll
  for (int u = 0; u < GATHER_UNROLL; ++u) {
    const int64_t r = r0 + u * GATHER_ROWS_PER_PASS;
    if (r < n)
      v[u] = load16_nt(pool + (uint64_t)slot[u] * KV_WIDTH + 16 * c);
  }
#pragma unroll
  for (int u = 0; u < GATHER_UNROLL; ++u) {
    const int64_t r = r0 + u * GATHER_ROWS_PER_PASS;
    if (r < n) {
      u32x4_t o0, o1;
      convert16(v[u], o0, o1);
      const int64_t j = 2 * (r * KV_CHUNKS + c);
      store16_nt(&out[j], o0);
      store16_nt(&out[j + 1], o1);
    }
  }
}

}  // namespace

hipError_t launch_cast_pool(const uint8_t* pool, int64_t num_slots, uint16_t* out,
                            hipStream_t stream, int num_cus) {
  const int64_t nchunks = num_slots * KV_CHUNKS;
  if (nchunks == 0) return hipSuccess;
  int64_t blocks = (nchunks + CAST_THREADS - 1) / CAST_THREADS;
  const int64_t cap = (int64_t)num_cus * 8;
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL(cast_pool_kernel, dim3((unsigned)blocks), dim3(CAST_THREADS), 0, stream,
                     reinterpret_cast<const u32x4_t*>(pool), reinterpret_cast<u32x4_t*>(out), nchunks);
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
