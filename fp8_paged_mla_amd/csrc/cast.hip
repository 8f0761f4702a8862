// FP8-E4M3FN -> BF16 cast kernels for gfx950: the full-pool cast and the
// gather-then-cast fallback.
//
// Both are pure bandwidth work (1 byte read, 2 bytes written per element, plus
// 4 index bytes per gathered row), so they are written for coalescing, not
// for arithmetic: every wave instruction covers one contiguous span, several
// loads are in flight per lane, and one conversion instruction handles two
// elements.
#include "decode_common.h"  // global->LDS copies and explicit vmcnt waits
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

// Full-pool cast.  The input reaches LDS by global->LDS copies, which keep
// more bytes in flight per CU than register loads do (no registers wait on
// them): each wave cycles through CAST_SLOTS private LDS slots of one
// 2 KB chunk each, copying chunk k + CAST_SLOTS while it converts and
// stores chunk k.  Chunks are dealt to waves grid-stride; lane l copies bytes
// 16l..16l+15 of each KB of the chunk and then reads back 8-byte pieces
// 512h + 8l (h = 0..3), so every store instruction writes 1 KB of
// contiguous BF16.  Only the issuing wave reads its slots, so an explicit
// vmcnt wait orders the copy before the reads.  The bytes past the last
// whole chunk are cast by the register path below.  One workgroup of four
// waves per CU with 4 KB in flight per wave measured fastest on MI355X.
constexpr int CAST_WAVES = 4;
constexpr int CAST_THREADS = 64 * CAST_WAVES;
constexpr int CAST_SLOTS = 2;
constexpr int CAST_CHUNK = 2048;                 // input bytes per chunk: two 1 KB copy ops
constexpr int CAST_OPS = CAST_CHUNK / 1024;

// Wait until chunk k of a wave's list (of K) has landed.  Issue order: the
// prologue copies chunks 0..P0-1 (P0 = min(K, CAST_SLOTS)); iteration j then
// issues the copies of chunk j + CAST_SLOTS (if any) and 2 * CAST_OPS stores,
// and stores count in vmcnt too.  The number of operations younger than
// chunk k's last copy is therefore
//   k < S:  OPS (P0 - 1 - k) + 3 OPS k - OPS m,
//   k >= S: 3 OPS (S - 1) + 2 OPS - OPS m,    m = #{j < k : j + S >= K},
// and waiting for at most the largest immediate below that count proves the
// chunk complete (a smaller immediate only waits longer).
__device__ __forceinline__ void cast_wait_chunk(int64_t k, int64_t K) {
  constexpr int S = CAST_SLOTS, OPS = CAST_OPS;
  const int64_t P0 = K < S ? K : S;
  const int64_t tail_start = K - S > 0 ? K - S : 0;
  const int64_t m = k > tail_start ? k - tail_start : 0;
  const int64_t younger = k < S ? OPS * (P0 - 1 - k) + 3 * OPS * k - OPS * m
                                : 3 * OPS * (S - 1) + 2 * OPS - OPS * m;
  using decode::wait_vm;
  if (younger >= 10) wait_vm<10>();
  else if (younger >= 8) wait_vm<8>();
  else if (younger >= 6) wait_vm<6>();
  else if (younger >= 4) wait_vm<4>();
  else if (younger >= 2) wait_vm<2>();
  else if (younger >= 1) wait_vm<1>();
  else wait_vm<0>();
}

__global__ __launch_bounds__(CAST_THREADS) void cast_pool_kernel(const uint8_t* __restrict__ in,
                                                                 u32x4_t* __restrict__ out,
                                                                 int64_t nbytes) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[CAST_WAVES][CAST_SLOTS][CAST_CHUNK];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t nchunks = nbytes / CAST_CHUNK;
  const int64_t gw = (int64_t)blockIdx.x * CAST_WAVES + w, nw = (int64_t)gridDim.x * CAST_WAVES;
  const int64_t K = gw < nchunks ? (nchunks - gw + nw - 1) / nw : 0;  // this wave's chunks
  const uint32_t base = (uint32_t)(uintptr_t)(
      (__attribute__((address_space(3))) uint8_t*)&ring[w][0][0]);
  auto issue_chunk = [&](int64_t k, int slot) {
    const uint8_t* src = in + (gw + k * nw) * CAST_CHUNK + 16 * lane;
#pragma unroll
    for (int o = 0; o < CAST_OPS; ++o)
      decode::issue_lds_dma16(src + 1024 * o,
                              __builtin_amdgcn_readfirstlane(base + CAST_CHUNK * slot + 1024 * o));
  };
  for (int d = 0; d < CAST_SLOTS; ++d)
    if (d < K) issue_chunk(d, d);
  for (int64_t k = 0; k < K; ++k) {
    cast_wait_chunk(k, K);
    const int slot = (int)(k % CAST_SLOTS);
    u32x2_t v[2 * CAST_OPS];
#pragma unroll
    for (int h = 0; h < 2 * CAST_OPS; ++h)
      v[h] = *reinterpret_cast<const u32x2_t*>(&ring[w][slot][512 * h + 8 * lane]);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the slot is read before it is refilled
    if (k + CAST_SLOTS < K) issue_chunk(k + CAST_SLOTS, slot);
    u32x4_t* dst = out + (gw + k * nw) * (CAST_CHUNK / 8) + lane;
#pragma unroll
    for (int h = 0; h < 2 * CAST_OPS; ++h) store16_nt(dst + 64 * h, convert8(v[h]));
  }
  decode::wait_vm<0>();
  // the bytes past the last whole chunk, 8 per lane, grid-stride
  const int64_t stride = (int64_t)gridDim.x * CAST_THREADS;
  for (int64_t i = nchunks * (CAST_CHUNK / 8) + (int64_t)blockIdx.x * CAST_THREADS + threadIdx.x;
       i < nbytes / 8; i += stride)
    store16_nt(&out[i], convert8(load8_nt(in + 8 * i)));
}

// Gather-then-cast.  Output rows go to waves in chunks of 16 consecutive
// rows (9 KB of FP8 in, 18 KB of BF16 out), grid-stride.  A chunk's slot ids
// and rows reach LDS by global->LDS copies: 64 bytes of ids into a small
// per-wave id ring, then 9 copy ops of 1 KB in which lane l of op j takes
// 16-byte piece P = 64j + l of the chunk (row P / 36, piece P % 36), so every
// op reads whole rows back to back.  The chunk is then read back linearly,
// 8 bytes per lane, converted and written with 18 contiguous 1 KB stores.
// Each wave keeps GATHER_SLOTS chunks in flight; the ids of chunk k + S + 1
// are copied one iteration before that chunk's rows.  No register is ever the
// destination of a load in flight.  Rows past the last whole chunk are cast
// by the register path below.
constexpr int GATHER_WAVES = 4;
constexpr int GATHER_THREADS = 64 * GATHER_WAVES;
constexpr int GATHER_SLOTS = 3;
constexpr int GATHER_ROWS = 16;                                 // rows per chunk
constexpr int GATHER_OPS = GATHER_ROWS * KV_WIDTH / 1024;       // 9 copy ops of 1 KB
constexpr int GATHER_STORES = GATHER_ROWS * KV_WIDTH * 2 / 1024;  // 18 stores of 1 KB
constexpr int GATHER_ID_SLOTS = GATHER_SLOTS + 2;
static_assert(GATHER_ROWS * KV_WIDTH == GATHER_OPS * 1024, "chunk is whole 1 KB copy ops");

// 4-byte global -> LDS copy (lane l's dword at lds_base + 4 l), with the wait
// state an LDS DMA needs after an M0 write.
__device__ __forceinline__ void issue_lds_dma4(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(g), "s"(lds_base)
               : "memory", "m0");
}

// Issue order of a wave with K chunks (S = GATHER_SLOTS, G = GATHER_OPS,
// R = GATHER_STORES): A = min(K, S + 1) id copies, one drain, the row copies of
// chunks 0..P0-1 (P0 = min(K, S)); then iteration j issues [ids of chunk
// j + S + 1, if any] [rows of chunk j + S, if any] [R stores].  With
// T(k) = T0 + sum over j < k of the ops of iteration j, waiting for at most
// min(younger than chunk k's last row copy, younger than chunk k + S's id
// copy) operations proves both complete (stores count in vmcnt too).
__device__ __forceinline__ void gather_wait_chunk(int64_t k, int64_t K) {
  constexpr int S = GATHER_SLOTS, G = GATHER_OPS, R = GATHER_STORES;
  const int64_t A = K < S + 1 ? K : S + 1;
  const int64_t P0 = K < S ? K : S;
  const int64_t T0 = A + G * P0;
  const int64_t KS = K - S > 0 ? K - S : 0, KS1 = K - S - 1 > 0 ? K - S - 1 : 0;
  auto ops_before = [&](int64_t i) -> int64_t {  // ops of iterations 0..i-1
    return R * i + G * (i < KS ? i : KS) + (i < KS1 ? i : KS1);
  };
  const int64_t Tk = T0 + ops_before(k);
  int64_t last_row_copy;
  if (k < P0) {
    last_row_copy = A + G * k + G - 1;
  } else {
    const int64_t j = k - S;
    last_row_copy = T0 + ops_before(j) + (j + S + 1 < K ? 1 : 0) + G - 1;
  }
  int64_t younger = Tk - last_row_copy - 1;
  if (k + S < K) {
    const int64_t id_copy = k == 0 ? S : T0 + ops_before(k - 1);
    const int64_t y = Tk - id_copy - 1;
    younger = y < younger ? y : younger;
  }
  using decode::wait_vm;
  if (younger >= 48) wait_vm<48>();
  else if (younger >= 40) wait_vm<40>();
  else if (younger >= 32) wait_vm<32>();
  else if (younger >= 27) wait_vm<27>();
  else if (younger >= 24) wait_vm<24>();
  else if (younger >= 18) wait_vm<18>();
  else if (younger >= 12) wait_vm<12>();
  else if (younger >= 9) wait_vm<9>();
  else if (younger >= 4) wait_vm<4>();
  else if (younger >= 1) wait_vm<1>();
  else wait_vm<0>();
}

__global__ __launch_bounds__(GATHER_THREADS) void gather_cast_kernel(
    const uint8_t* __restrict__ pool, uint32_t max_slot, const int32_t* __restrict__ indices,
    int64_t n, u32x4_t* __restrict__ out) {
  constexpr int S = GATHER_SLOTS;
  __shared__ __attribute__((aligned(16))) uint8_t ring[GATHER_WAVES][S][GATHER_OPS * 1024];
  __shared__ __attribute__((aligned(16))) int32_t id_ring[GATHER_WAVES][GATHER_ID_SLOTS][64];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t nchunks = n / GATHER_ROWS;
  const int64_t gw = (int64_t)blockIdx.x * GATHER_WAVES + w, nw = (int64_t)gridDim.x * GATHER_WAVES;
  const int64_t K = gw < nchunks ? (nchunks - gw + nw - 1) / nw : 0;  // this wave's chunks
  const uint32_t rows_base = (uint32_t)(uintptr_t)(
      (__attribute__((address_space(3))) uint8_t*)&ring[w][0][0]);
  const uint32_t ids_base = (uint32_t)(uintptr_t)(
      (__attribute__((address_space(3))) int32_t*)&id_ring[w][0][0]);
  // slot ids of chunk k (lane l copies row l & 15) into id slot k % GATHER_ID_SLOTS
  auto copy_ids = [&](int64_t k) -> int {
    const int slot = (int)(k % GATHER_ID_SLOTS);
    issue_lds_dma4(indices + (gw + k * nw) * GATHER_ROWS + (lane & 15),
                   __builtin_amdgcn_readfirstlane(ids_base + 256 * slot));
    return slot;
  };
  auto copy_rows = [&](int id_slot, int slot) {
#pragma unroll
    for (int j = 0; j < GATHER_OPS; ++j) {
      const int P = 64 * j + lane;
      const int r = P / KV_CHUNKS;
      const uint32_t s = (uint32_t)id_ring[w][id_slot][r];  // negative ids compare as large
      const uint8_t* src = pool + (uint64_t)(s < max_slot ? s : max_slot) * KV_WIDTH +
                           16 * (P - KV_CHUNKS * r);
      decode::issue_lds_dma16_nt(src, __builtin_amdgcn_readfirstlane(
                                       rows_base + GATHER_OPS * 1024 * slot + 1024 * j));
    }
  };

  const int64_t A = K < S + 1 ? K : S + 1;
  const int64_t P0 = K < S ? K : S;
  int id_slot[S + 1];
#pragma unroll
  for (int d = 0; d <= S; ++d) id_slot[d] = d < A ? copy_ids(d) : 0;
  decode::wait_vm<0>();
#pragma unroll
  for (int d = 0; d < S; ++d)
    if (d < P0) copy_rows(id_slot[d], d);
  int ids_next = id_slot[S];
  for (int64_t k = 0; k < K; ++k) {
    gather_wait_chunk(k, K);
    const int slot = (int)(k % S);
    u32x2_t v[GATHER_STORES];
#pragma unroll
    for (int h = 0; h < GATHER_STORES; ++h)
      v[h] = *reinterpret_cast<const u32x2_t*>(&ring[w][slot][512 * h + 8 * lane]);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the slot is read before it is refilled
    if (k + S < K) {
      const int ids = ids_next;
      if (k + S + 1 < K) ids_next = copy_ids(k + S + 1);
      copy_rows(ids, slot);
    }
    u32x4_t* dst = out + (gw + k * nw) * GATHER_ROWS * (KV_WIDTH / 8) + lane;
#pragma unroll
    for (int h = 0; h < GATHER_STORES; ++h) store16_dev(dst + 64 * h, convert8(v[h]));
  }
  decode::wait_vm<0>();
  // rows past the last whole chunk, 8 bytes per lane
  const int64_t first = nchunks * GATHER_ROWS * (KV_WIDTH / 8);
  const int64_t total = n * (KV_WIDTH / 8);
  for (int64_t e = first + (int64_t)blockIdx.x * GATHER_THREADS + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * GATHER_THREADS) {
    const int64_t r = e / (KV_WIDTH / 8);
    const int c = (int)(e - r * (KV_WIDTH / 8));
    const uint32_t s = (uint32_t)indices[r];
    store16_dev(&out[e], convert8(load8_nt(pool + (uint64_t)(s < max_slot ? s : max_slot) * KV_WIDTH + 8 * c)));
  }
}

}  // namespace

hipError_t launch_cast_pool(const uint8_t* pool, int64_t num_slots, uint16_t* out,
                            hipStream_t stream, int num_cus) {
  const int64_t nbytes = num_slots * KV_WIDTH;  // a multiple of 64
  if (nbytes == 0) return hipSuccess;
  // one workgroup per CU (fewer for pools of fewer chunks than waves)
  const int64_t waves_needed = nbytes / CAST_CHUNK + 1;
  int64_t blocks = (waves_needed + CAST_WAVES - 1) / CAST_WAVES;
  if (blocks > num_cus) blocks = num_cus;
  hipLaunchKernelGGL(cast_pool_kernel, dim3((unsigned)blocks), dim3(CAST_THREADS), 0, stream,
                     pool, reinterpret_cast<u32x4_t*>(out), nbytes);
  return hipGetLastError();
}

hipError_t launch_gather_cast(const uint8_t* pool, int64_t num_slots, const int32_t* indices,
                              int64_t n, uint16_t* out, hipStream_t stream, int num_cus) {
  if (n == 0) return hipSuccess;
  // one workgroup per CU (fewer when there are fewer chunks than waves)
  const int64_t waves_needed = n / GATHER_ROWS + 1;
  int64_t blocks = (waves_needed + GATHER_WAVES - 1) / GATHER_WAVES;
  if (blocks > num_cus) blocks = num_cus;
  hipLaunchKernelGGL(gather_cast_kernel, dim3((unsigned)blocks), dim3(GATHER_THREADS), 0, stream,
                     pool, (uint32_t)(num_slots - 1), indices, n, reinterpret_cast<u32x4_t*>(out));
  return hipGetLastError();
}

}  // namespace fp8mla
