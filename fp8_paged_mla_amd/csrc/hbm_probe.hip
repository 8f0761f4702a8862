// HBM ceiling probes for gfx950: plain streams and a random-row gather that
// measure what this device's memory system delivers for the access mixes
// the library's kernels use, so that each kernel's bandwidth can be stated
// against a measured ceiling as well as the 8 TB/s specification ("The KV
// Cache Cast Bottleneck", Reasoning: the cast's efficiency is judged against
// the device's bandwidth).  Benchmark-only; none of the library's paths call
// them.
//  * read:   a sequential stream, loads only (the attention's reads);
//  * copy12: a sequential stream reading 1 byte for every 2 written (the
//            FP8 -> BF16 cast's mix);
//  * write:  a sequential stream, stores only (the cast's write side);
//  * gather: 576-byte rows at random slots copied global -> LDS by 16-byte
//            copies, whole rows back to back, with 1 or 2 chunks of 16 rows
//            in flight per wave and no arithmetic (the decode's row gather
//            without its math).
#include "decode_common.h"  // LDS copies, explicit vmcnt waits
#include "launch.h"

namespace fp8mla {
namespace {

constexpr int PROBE_THREADS = 256;
constexpr uint32_t kNever = 0x9E3779B9u;  // the sink is written only if a checksum equals this

template <int U>
__global__ __launch_bounds__(PROBE_THREADS) void probe_read_kernel(const u32x4_t* __restrict__ src,
                                                                   int64_t nchunks,
                                                                   uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const int64_t step = (int64_t)gridDim.x * PROBE_THREADS * U;
  for (int64_t base = (int64_t)blockIdx.x * PROBE_THREADS * U + threadIdx.x; base < nchunks;
       base += step) {
    u32x4_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + (int64_t)PROBE_THREADS * u;
      v[u] = i < nchunks ? load16_nt(src + i) : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  if (acc == kNever) sink[blockIdx.x] = acc;  // keeps the loads; never true for the probe's data
}

// Every 16-byte chunk of src is written twice into dst: 1 byte read per 2
// written.  A wave reads 64 consecutive chunks (1 KB) and writes them to the
// corresponding 2 KB of dst, twice, in two contiguous 1 KB stores.
template <int U>
__global__ __launch_bounds__(PROBE_THREADS) void probe_copy12_kernel(const u32x4_t* __restrict__ src,
                                                                     int64_t nchunks,
                                                                     u32x4_t* __restrict__ dst) {
  const int64_t step = (int64_t)gridDim.x * PROBE_THREADS * U;
  for (int64_t base = (int64_t)blockIdx.x * PROBE_THREADS * U + threadIdx.x; base < nchunks;
       base += step) {
    u32x4_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + (int64_t)PROBE_THREADS * u;
      v[u] = i < nchunks ? load16_nt(src + i) : u32x4_t{0u, 0u, 0u, 0u};
    }
    const int l = threadIdx.x & 63;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + (int64_t)PROBE_THREADS * u;
      if (i < nchunks) {
        // the wave's 64 chunks (1 KB read) go to 128 chunks of dst (2 KB),
        // written by two stores that each cover one contiguous 1 KB span
        u32x4_t* d = dst + 2 * (i - l) + l;
        store16_nt(d, v[u]);
        store16_nt(d + 64, v[u]);
      }
    }
  }
}

// Sequential writes only: a constant pattern stored in contiguous 1 KB wave
// spans (the write side of the cast's mix).
template <int U>
__global__ __launch_bounds__(PROBE_THREADS) void probe_write_kernel(u32x4_t* __restrict__ dst,
                                                                    int64_t nchunks) {
  const int64_t step = (int64_t)gridDim.x * PROBE_THREADS * U;
  const u32x4_t v = {0x3C3C3C3Cu, 0x3C3C3C3Cu, 0x3C3C3C3Cu, (uint32_t)threadIdx.x};
  for (int64_t base = (int64_t)blockIdx.x * PROBE_THREADS * U + threadIdx.x; base < nchunks;
       base += step) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + (int64_t)PROBE_THREADS * u;
      if (i < nchunks) store16_nt(dst + i, v);
    }
  }
}

// Random-row gather into LDS.  Chunk c = rows 16c .. 16c+15 of the index
// list; wave g of the grid takes chunks g, g + nw, g + 2 nw, ...  A chunk is
// 10 global->LDS copy ops (16 rows x 37 16-byte LDS slots: 36 data chunks and
// a pad, an odd stride), lane l of op j taking LDS slot 64 j + l = row P / 37,
// chunk P % 37 (the pad slot re-reads chunk 35), as the decode copies a tile.
// S chunks per wave are in flight: chunk k + S is copied as soon as chunk k
// has been read back.  Slot ids are loaded S chunks ahead.
constexpr int G_WAVES = 8;
constexpr int G_ROW_SLOTS = KV_CHUNKS + 1;              // 37
constexpr int G_CHUNK_LDS = 16 * 16 * G_ROW_SLOTS;      // 9472 bytes
constexpr int G_OPS = (16 * G_ROW_SLOTS + 63) / 64;     // 10

template <int S>
__global__ __launch_bounds__(64 * G_WAVES) void probe_gather_kernel(const uint8_t* __restrict__ pool,
                                                                    uint32_t max_slot,
                                                                    const int32_t* __restrict__ idx,
                                                                    int64_t nchunks,
                                                                    uint32_t* __restrict__ sink) {
  static_assert(S == 1 || S == 2, "one or two chunks in flight per wave");
  __shared__ __attribute__((aligned(16))) uint8_t lds[G_WAVES][S][G_CHUNK_LDS];
  using namespace decode;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t gw = (int64_t)blockIdx.x * G_WAVES + w, nw = (int64_t)gridDim.x * G_WAVES;
  const int64_t K = gw < nchunks ? (nchunks - gw + nw - 1) / nw : 0;
  const uint32_t base = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint8_t*)&lds[w][0][0]);
  // slot id of row (lane & 15) of this wave's chunk k; past the wave's last
  // chunk the load reads entry 0 (in bounds, unused)
  auto load_ids = [&](int64_t k) -> int32_t {
    const int64_t row = k < K ? 16 * (gw + k * nw) + (lane & 15) : 0;
    return issue_load_i32(idx + row);
  };
  auto issue_rows = [&](int slot, int32_t ix) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int j = 0; j < G_OPS; ++j) {
      const int P = 64 * j + ln;
      const int r = P / G_ROW_SLOTS;
      const int c = min(P - r * G_ROW_SLOTS, KV_CHUNKS - 1);
      const uint32_t s = (uint32_t)__shfl(ix, r & 15);
      const uint8_t* a = pool + (uint64_t)(s < max_slot ? s : max_slot) * KV_WIDTH + 16 * c;
      if (j < G_OPS - 1 || P < 16 * G_ROW_SLOTS)
        issue_lds_dma16_nt(a, __builtin_amdgcn_readfirstlane(base + slot * G_CHUNK_LDS + 1024 * j));
    }
  };
  uint32_t acc = 0;
  auto consume = [&](int slot) {
    acc ^= *reinterpret_cast<const uint32_t*>(&lds[w][slot][16 * lane]);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // read back before the slot is refilled
  };
  if constexpr (S == 1) {
    // Issue order per chunk k: rows(k), ids(k+1).  Top of iteration k:
    // rows(k) then ids(k+1) outstanding.
    int32_t ix = load_ids(0);
    wait_vm<0>();
    pin(ix);
    if (K > 0) issue_rows(0, ix);
    ix = load_ids(1);
    for (int64_t k = 0; k < K; ++k) {
      wait_vm<1>();  // rows(k) landed (younger: ids(k+1))
      consume(0);
      wait_vm<0>();  // ids(k+1)
      pin(ix);
      if (k + 1 < K) issue_rows(0, ix);
      ix = load_ids(k + 2);
    }
  } else {
    // Issue order: rows(k), ids(k+2), rows(k+1), ids(k+3), ...  At the top
    // of iteration k the ops younger than rows(k) are ids(k+2), rows(k+1) if
    // k + 1 < K, ids(k+3).
    int32_t ixA = load_ids(0), ixB = load_ids(1);  // ixA: even chunks, ixB: odd chunks
    wait_vm<0>();
    pin(ixA);
    pin(ixB);
    if (K > 0) issue_rows(0, ixA);
    ixA = load_ids(2);
    if (K > 1) issue_rows(1, ixB);
    ixB = load_ids(3);
    auto step = [&](int64_t k, int32_t& ix_cur) {
      if (k + 1 < K) wait_vm<12>();
      else wait_vm<2>();
      consume((int)(k & 1));
      if (k + 1 < K) wait_vm<11>();  // ids(k+2) (younger: rows(k+1), ids(k+3))
      else wait_vm<1>();
      pin(ix_cur);
      if (k + 2 < K) issue_rows((int)(k & 1), ix_cur);
      ix_cur = load_ids(k + 4);
    };
    for (int64_t k = 0; k < K; k += 2) {
      step(k, ixA);
      if (k + 1 >= K) break;
      step(k + 1, ixB);
    }
  }
  wait_vm<0>();
  if (acc == kNever) sink[gw] = acc;
}

}  // namespace

hipError_t launch_probe_read(const void* src, int64_t bytes, int grid, int unroll, uint32_t* sink,
                             hipStream_t stream) {
  const u32x4_t* s = reinterpret_cast<const u32x4_t*>(src);
  const int64_t n = bytes / 16;
  switch (unroll) {
    case 4: hipLaunchKernelGGL(probe_read_kernel<4>, dim3(grid), dim3(PROBE_THREADS), 0, stream, s, n, sink); break;
    case 8: hipLaunchKernelGGL(probe_read_kernel<8>, dim3(grid), dim3(PROBE_THREADS), 0, stream, s, n, sink); break;
    default: hipLaunchKernelGGL(probe_read_kernel<16>, dim3(grid), dim3(PROBE_THREADS), 0, stream, s, n, sink); break;
  }
  return hipGetLastError();
}

hipError_t launch_probe_copy12(const void* src, int64_t bytes, void* dst, int grid, int unroll,
                               hipStream_t stream) {
  const u32x4_t* s = reinterpret_cast<const u32x4_t*>(src);
  u32x4_t* d = reinterpret_cast<u32x4_t*>(dst);
  const int64_t n = bytes / 16;
  switch (unroll) {
    case 4: hipLaunchKernelGGL(probe_copy12_kernel<4>, dim3(grid), dim3(PROBE_THREADS), 0, stream, s, n, d); break;
    case 8: hipLaunchKernelGGL(probe_copy12_kernel<8>, dim3(grid), dim3(PROBE_THREADS), 0, stream, s, n, d); break;
    default: hipLaunchKernelGGL(probe_copy12_kernel<16>, dim3(grid), dim3(PROBE_THREADS), 0, stream, s, n, d); break;
  }
  return hipGetLastError();
}

hipError_t launch_probe_write(void* dst, int64_t bytes, int grid, int unroll, hipStream_t stream) {
  u32x4_t* d = reinterpret_cast<u32x4_t*>(dst);
  const int64_t n = bytes / 16;
  switch (unroll) {
    case 4: hipLaunchKernelGGL(probe_write_kernel<4>, dim3(grid), dim3(PROBE_THREADS), 0, stream, d, n); break;
    case 8: hipLaunchKernelGGL(probe_write_kernel<8>, dim3(grid), dim3(PROBE_THREADS), 0, stream, d, n); break;
    default: hipLaunchKernelGGL(probe_write_kernel<16>, dim3(grid), dim3(PROBE_THREADS), 0, stream, d, n); break;
  }
  return hipGetLastError();
}

hipError_t launch_probe_gather(const uint8_t* pool, int64_t num_slots, const int32_t* idx,
                               int64_t n, int grid, int chunks_in_flight, uint32_t* sink,
                               hipStream_t stream) {
  const uint32_t max_slot = (uint32_t)(num_slots - 1);
  const int64_t nchunks = n / 16;
  if (chunks_in_flight == 1)
    hipLaunchKernelGGL(probe_gather_kernel<1>, dim3(grid), dim3(64 * G_WAVES), 0, stream, pool,
                       max_slot, idx, nchunks, sink);
  else
    hipLaunchKernelGGL(probe_gather_kernel<2>, dim3(grid), dim3(64 * G_WAVES), 0, stream, pool,
                       max_slot, idx, nchunks, sink);
  return hipGetLastError();
}

}  // namespace fp8mla

// ---- C ABI (declared in include/fp8mla_probe.h)
#include "../../include/fp8mla.h"
#include "../../include/fp8mla_probe.h"

namespace {
bool probe_aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool probe_grid_ok(int32_t grid) { return grid >= 1 && grid <= 65536; }
bool probe_unroll_ok(int32_t u) { return u == 4 || u == 8 || u == 16; }
}  // namespace

extern "C" {

int fp8mla_probe_read(const void* src, int64_t bytes, int32_t grid, int32_t unroll, uint32_t* sink,
                      void* stream) {
  if (bytes <= 0 || bytes % 16 != 0 || !probe_grid_ok(grid) || !probe_unroll_ok(unroll))
    return FP8MLA_ERR_BAD_SHAPE;
  if (!src || !sink) return FP8MLA_ERR_NULL_PTR;
  if (!probe_aligned16(src)) return FP8MLA_ERR_MISALIGNED;
  return fp8mla::launch_probe_read(src, bytes, grid, unroll, sink,
                                   static_cast<hipStream_t>(stream)) == hipSuccess
             ? FP8MLA_OK
             : FP8MLA_ERR_HIP;
}

int fp8mla_probe_copy_1to2(const void* src, int64_t bytes, void* dst, int32_t grid, int32_t unroll,
                           void* stream) {
  // whole 1 KB wave spans: every wave's 64 chunks are all in range or all out
  if (bytes <= 0 || bytes % 1024 != 0 || !probe_grid_ok(grid) || !probe_unroll_ok(unroll))
    return FP8MLA_ERR_BAD_SHAPE;
  if (!src || !dst) return FP8MLA_ERR_NULL_PTR;
  if (!probe_aligned16(src) || !probe_aligned16(dst)) return FP8MLA_ERR_MISALIGNED;
  return fp8mla::launch_probe_copy12(src, bytes, dst, grid, unroll,
                                     static_cast<hipStream_t>(stream)) == hipSuccess
             ? FP8MLA_OK
             : FP8MLA_ERR_HIP;
}

int fp8mla_probe_write(void* dst, int64_t bytes, int32_t grid, int32_t unroll, void* stream) {
  if (bytes <= 0 || bytes % 16 != 0 || !probe_grid_ok(grid) || !probe_unroll_ok(unroll))
    return FP8MLA_ERR_BAD_SHAPE;
  if (!dst) return FP8MLA_ERR_NULL_PTR;
  if (!probe_aligned16(dst)) return FP8MLA_ERR_MISALIGNED;
  return fp8mla::launch_probe_write(dst, bytes, grid, unroll, static_cast<hipStream_t>(stream)) ==
                 hipSuccess
             ? FP8MLA_OK
             : FP8MLA_ERR_HIP;
}

int fp8mla_probe_gather_rows(const uint8_t* pool, int64_t num_slots, const int32_t* indices,
                             int64_t n, int32_t grid, int32_t chunks_in_flight, uint32_t* sink,
                             void* stream) {
  if (num_slots < 1 || num_slots > (int64_t)UINT32_MAX || n < 16 || n % 16 != 0 ||
      n > (int64_t)INT32_MAX || !probe_grid_ok(grid) ||
      (chunks_in_flight != 1 && chunks_in_flight != 2))
    return FP8MLA_ERR_BAD_SHAPE;
  if (!pool || !indices || !sink) return FP8MLA_ERR_NULL_PTR;
  if (!probe_aligned16(pool) || (reinterpret_cast<uintptr_t>(indices) & 3u) != 0)
    return FP8MLA_ERR_MISALIGNED;
  return fp8mla::launch_probe_gather(pool, num_slots, indices, n, grid, chunks_in_flight, sink,
                                     static_cast<hipStream_t>(stream)) == hipSuccess
             ? FP8MLA_OK
             : FP8MLA_ERR_HIP;
}

}  // extern "C"
