// Split-K MLA decode over a paged FP8-E4M3FN latent cache, for gfx950.
//
// What is computed (per request b, query head h; one KV head shared by all
// heads; 576 = 512 latent + 64 rope as in "The KV Cache Cast Bottleneck",
// The Context):
//   s[t] = sm_scale * scale * <q[b,h,:576], e4m3(row_t[:576])>
//   out[b,h,:] = scale * sum_t softmax(s)[t] * e4m3(row_t[:512])
// Only the rows named by kv_indices are read, and they are dequantised in the
// kernel: the fix the pages call for instead of the full-pool .to() cast.
//
// Work decomposition.  The concatenated token stream of all requests
// (length N = kv_indptr[B]) is cut into equal segments; one workgroup
// processes one segment for one group of 16 heads, walking it in tiles of
// 128 tokens and handling request boundaries inside the tile.  For every
// request it touches it writes either the final output (request entirely
// inside the segment) or a partial (o normalised, log2-sum-exp) that the
// combine kernel merges.  Segments are balanced by tokens, not by request,
// so long and short requests cost the same per token.
//
// Inside a workgroup (8 waves, 16 heads):
//  * wave w owns tokens [16w, 16w+16) of each tile for the score product
//    S^T = K q^T (MFMA 16x16x32 bf16, M = 16 tokens, N = 16 heads,
//    K = 576 in 18 steps).  Its lanes load those tokens' 576-byte rows with
//    16-byte loads straight into registers, already in MFMA A-operand order
//    (lane (t, g) holds 16 bytes at offset 64*i + 16*g of row t), two tiles
//    ahead of use; the FP8 bytes are converted to bf16 right before the MFMA.
//  * the same registers hold the value part (first 512 bytes) of each row;
//    they are written once to LDS, where every wave reads the transposed
//    operand it needs with ds_read_b64_tr_b8.
//  * the softmax is exchanged through LDS: wave-local maxima, then bf16
//    probabilities; all waves then share one running maximum per head.
//  * wave w owns output columns [64w, 64w+64) of the P.V product
//    O^T = V^T P^T (MFMA 16x16x32 bf16, M = 16 columns, N = 16 heads,
//    K = 32 tokens), so no cross-wave reduction of O is needed.
// KV bytes move from HBM exactly once per head group; every value byte is
// converted once per wave that consumes it.
#include "device_common.h"
#include "launch.h"

#include <math.h>

namespace fp8mla {
namespace {

constexpr int NWAVES = 8;
constexpr int THREADS = 64 * NWAVES;              // 512
constexpr int TILE = 16 * NWAVES;                 // tokens per tile: 16 per wave
constexpr int HEADS = 16;                         // heads per workgroup
constexpr int ROWB = KV_WIDTH + 16;               // LDS bytes per row: 37 16-byte slots (odd stride)
constexpr int TILE_BYTES = TILE * ROWB;           // 75776
constexpr int KCHUNKS = KV_WIDTH / 64;            // 16-byte loads per lane per tile; query steps / 2
constexpr int QPIECES = 2 * KCHUNKS * 64;         // 16-byte pieces of one head group's query

struct SplitParams {
  const uint16_t* q;
  const uint8_t* pool;
  const int32_t* indptr;
  const int32_t* indices;
  uint16_t* out;
  float* part_o;
  float* part_lse;
  uint32_t max_slot;
  int32_t total_tokens;
  int32_t B;
  int32_t H;
  int32_t HG;
  int32_t Hp;
  int32_t seg_len;
  int32_t items;
  int32_t xcd_per;
  float score_scale;  // sm_scale * scale * log2(e): scores in the base-2 domain
  float kv_scale;
};

struct CombineParams {
  const int32_t* indptr;
  const float* part_o;
  const float* part_lse;
  uint16_t* out;
  int32_t total_tokens;
  int32_t B;
  int32_t H;
  int32_t Hp;
  int32_t seg_len;
  float kv_scale;
};

__device__ __forceinline__ float wave_max_over_groups(float x) {
  // lanes h, h+16, h+32, h+48 hold the same head
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

__device__ __forceinline__ float wave_sum_over_groups(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

__device__ __forceinline__ int clamp_tok(int v, int n) { return v < 0 ? 0 : (v > n ? n : v); }

// Byte mask over 4 consecutive tokens base..base+3: 0xFF for each token in
// [lo, hi), 0 otherwise.
__device__ __forceinline__ uint32_t run_mask(int base, int lo, int hi) {
  const int a = min(max(lo - base, 0), 4);
  const int b = min(max(hi - base, 0), 4);
  if (b <= a) return 0u;
  const uint64_t upto_b = (b == 4) ? 0xFFFFFFFFull : ((1ull << (8 * b)) - 1ull);
  const uint64_t below_a = (1ull << (8 * a)) - 1ull;
  return (uint32_t)(upto_b & ~below_a);
}

// ---- explicitly pipelined loads.  The row and index loads of the tile
// pipeline are issued as inline assembly and waited for with an explicit
// s_waitcnt vmcnt(N): left to itself the compiler sinks prefetches down to
// their first use (or drains every load at the loop head), which removes the
// overlap the register ring exists for.  Vector-memory operations complete
// in issue order, so "at most N outstanding" proves every older load done.
// After a wait, pin() makes the compiler treat the registers as redefined
// there, so no use of the data can be scheduled above the wait.
__device__ __forceinline__ int32_t issue_load_i32(const int32_t* p) {
  int32_t v;
  asm volatile("global_load_dword %0, %1, off" : "=v"(v) : "v"(p));
  return v;
}

__device__ __forceinline__ void issue_load_rows(u32x4_t (&kb)[9], const uint8_t* const (&a)[9]) {
  asm volatile(
      "global_load_dwordx4 %0, %9, off nt\n\t"
      "global_load_dwordx4 %1, %10, off nt\n\t"
      "global_load_dwordx4 %2, %11, off nt\n\t"
      "global_load_dwordx4 %3, %12, off nt\n\t"
      "global_load_dwordx4 %4, %13, off nt\n\t"
      "global_load_dwordx4 %5, %14, off nt\n\t"
      "global_load_dwordx4 %6, %15, off nt\n\t"
      "global_load_dwordx4 %7, %16, off nt\n\t"
      "global_load_dwordx4 %8, %17, off nt"
      : "=&v"(kb[0]), "=&v"(kb[1]), "=&v"(kb[2]), "=&v"(kb[3]), "=&v"(kb[4]), "=&v"(kb[5]),
        "=&v"(kb[6]), "=&v"(kb[7]), "=&v"(kb[8])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]),
        "v"(a[8]));
}

// Query operand of one lane: 9 pairs of 16-byte pieces 64 elements (128
// bytes) apart.
__device__ __forceinline__ void issue_load_q(bf16x8_t (&q)[18], const uint16_t* qp) {
  asm volatile(
      "global_load_dwordx4 %0, %18, off\n\t"
      "global_load_dwordx4 %1, %18, off offset:16\n\t"
      "global_load_dwordx4 %2, %18, off offset:128\n\t"
      "global_load_dwordx4 %3, %18, off offset:144\n\t"
      "global_load_dwordx4 %4, %18, off offset:256\n\t"
      "global_load_dwordx4 %5, %18, off offset:272\n\t"
      "global_load_dwordx4 %6, %18, off offset:384\n\t"
      "global_load_dwordx4 %7, %18, off offset:400\n\t"
      "global_load_dwordx4 %8, %18, off offset:512\n\t"
      "global_load_dwordx4 %9, %18, off offset:528\n\t"
      "global_load_dwordx4 %10, %18, off offset:640\n\t"
      "global_load_dwordx4 %11, %18, off offset:656\n\t"
      "global_load_dwordx4 %12, %18, off offset:768\n\t"
      "global_load_dwordx4 %13, %18, off offset:784\n\t"
      "global_load_dwordx4 %14, %18, off offset:896\n\t"
      "global_load_dwordx4 %15, %18, off offset:912\n\t"
      "global_load_dwordx4 %16, %18, off offset:1024\n\t"
      "global_load_dwordx4 %17, %18, off offset:1040"
      : "=&v"(q[0]), "=&v"(q[1]), "=&v"(q[2]), "=&v"(q[3]), "=&v"(q[4]), "=&v"(q[5]), "=&v"(q[6]),
        "=&v"(q[7]), "=&v"(q[8]), "=&v"(q[9]), "=&v"(q[10]), "=&v"(q[11]), "=&v"(q[12]),
        "=&v"(q[13]), "=&v"(q[14]), "=&v"(q[15]), "=&v"(q[16]), "=&v"(q[17])
      : "v"(qp));
}

__device__ __forceinline__ void pin_q(bf16x8_t (&q)[18]) {
  asm volatile(""
               : "+v"(q[0]), "+v"(q[1]), "+v"(q[2]), "+v"(q[3]), "+v"(q[4]), "+v"(q[5]),
                 "+v"(q[6]), "+v"(q[7]), "+v"(q[8]));
  asm volatile(""
               : "+v"(q[9]), "+v"(q[10]), "+v"(q[11]), "+v"(q[12]), "+v"(q[13]), "+v"(q[14]),
                 "+v"(q[15]), "+v"(q[16]), "+v"(q[17]));
}

__device__ __forceinline__ u32x4_t issue_load_16(const void* p) {
  u32x4_t v;
  asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(v) : "v"(p));
  return v;
}

// Global -> LDS copy of 16 bytes per lane: lane l's bytes land at LDS byte
// address lds_base + 16*l (lds_base wave-uniform, passed in M0).  Issued as
// inline assembly so that the compiler neither drains it at barriers nor
// waits for it before unrelated LDS reads; the caller waits with vmcnt.
// M0 is not otherwise used by these kernels.
__device__ __forceinline__ void issue_lds_dma16(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(lds_base)
               : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N));
}

__device__ __forceinline__ void pin(u32x4_t (&kb)[9]) {
  asm volatile(""
               : "+v"(kb[0]), "+v"(kb[1]), "+v"(kb[2]), "+v"(kb[3]), "+v"(kb[4]), "+v"(kb[5]),
                 "+v"(kb[6]), "+v"(kb[7]), "+v"(kb[8]));
}

__device__ __forceinline__ void pin(int32_t& x) { asm volatile("" : "+v"(x)); }

__device__ __forceinline__ void pin(u32x4_t& x) { asm volatile("" : "+v"(x)); }

// Token row (tile-relative) held by MFMA row m of wave w.  Odd waves use
// row m ^ 12 so that the transposed LDS reads of two consecutive waves'
// rows fall in distinct banks.
__device__ __forceinline__ int tile_row(int w, int m) { return 16 * w + ((w & 1) ? (m ^ 12) : m); }

__global__ __launch_bounds__(THREADS) void mla_split_kernel(const SplitParams p) {
  // One row tile, the query of the current request, and the softmax exchange.
  __shared__ __attribute__((aligned(16))) uint8_t kv_lds[TILE_BYTES];
  __shared__ u32x4_t q_lds[2][2 * KCHUNKS][64];  // current query and the next request's
  __shared__ float mx_lds[NWAVES][HEADS];
  __shared__ uint2 p_lds[NWAVES][64];
  __shared__ float l_lds[NWAVES][HEADS];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t = lane & 15;  // MFMA row/column index inside the 16-lane group
  const int g = lane >> 4;  // 16-lane group

  int item = blockIdx.x;
  if (p.HG > 1) item = (int)(blockIdx.x & 7) * p.xcd_per + (int)(blockIdx.x >> 3);
  if (item >= p.items) return;
  const int seg = item / p.HG;
  const int hg = item - seg * p.HG;
  const int N = p.total_tokens;
  const int seg_lo = seg * p.seg_len;
  const int seg_hi = min(N, seg_lo + p.seg_len);
  if (seg_lo >= seg_hi) return;
  const int ntiles = (seg_hi - seg_lo + TILE - 1) / TILE;
  const int head = hg * HEADS + t;  // head whose scores / outputs this lane carries

  // ---- loads.  Wave w fetches rows 16w..16w+15 of each tile.  Its 16 x 36
  // chunks of 16 bytes are numbered P = 36*r + c and lane l takes P = 64j + l
  // in load j (j < 9): each load instruction reads whole rows back to back
  // (one contiguous run per row, ~1.8 rows per instruction), the pattern that
  // gathers random 576-byte rows fastest.  Lanes r < 16 (and their copies at
  // r + 16k) hold the slot id of row r; each load gets its row's slot with a
  // cross-lane permute.  A lane whose token lies past the segment reads the
  // segment's first row instead (a cache hit); its scores and value bytes
  // are masked out.
  auto opaque_lane = [&]() -> int {  // recomputed per use, not kept across the loop
    int l = lane;
    asm volatile("" : "+v"(l));
    return l;
  };
  auto load_index = [&](int k) -> int32_t {
    const int tok = seg_lo + k * TILE + 16 * w + t;
    return issue_load_i32(p.indices + (tok < seg_hi ? tok : seg_lo));
  };
  auto load_rows = [&](int32_t idx, u32x4_t (&kb)[KCHUNKS]) {
    const uint8_t* a[KCHUNKS];
    const int ln = opaque_lane();
#pragma unroll
    for (int j = 0; j < KCHUNKS; ++j) {
      const int P = 64 * j + ln;
      const int r = P / KV_CHUNKS;
      const int c = P - r * KV_CHUNKS;
      const uint32_t s = (uint32_t)__shfl(idx, r);
      a[j] = p.pool + (uint64_t)(s < p.max_slot ? s : p.max_slot) * KV_WIDTH + 16 * c;
    }
    issue_load_rows(kb, a);
  };
  // stage a tile's rows (this wave's 16) into the LDS row tile
  auto store_rows = [&](const u32x4_t (&kb)[KCHUNKS]) {
    const int ln = opaque_lane();
#pragma unroll
    for (int j = 0; j < KCHUNKS; ++j) {
      const int P = 64 * j + ln;
      const int r = P / KV_CHUNKS;
      *reinterpret_cast<u32x4_t*>(kv_lds + (16 * w + r) * ROWB + 16 * (P - r * KV_CHUNKS)) = kb[j];
    }
  };

  u32x4_t kb0[KCHUNKS], kb1[KCHUNKS], kb2[KCHUNKS];
  int32_t ix0 = load_index(0);
  int32_t ix1 = load_index(1);
  int32_t ix2 = load_index(2);

  // ---- first request touching the segment: number of requests ending at or
  // before seg_lo.  Lane j of a 64-entry window holds kv_indptr[win + j];
  // for batches up to 63 one load covers the whole array, otherwise a
  // coarse-then-fine search over kv_indptr[1..B] (64 samples per round) runs
  // first.  Requests with no tokens are skipped by construction.
  int cur_b;
  int win = 0;
  int win_val;
  if (p.B <= 63) {
    win_val = clamp_tok(p.indptr[min(lane, p.B)], N);
    cur_b = __popcll(__ballot(lane >= 1 && lane <= p.B && win_val <= seg_lo));
  } else {
    int lo = 0, n = p.B;
    while (n > 64) {
      const int stride = (n + 63) / 64;
      const int j = lo + lane * stride;
      const bool le = j < lo + n && clamp_tok(p.indptr[j + 1], N) <= seg_lo;
      const int c = __popcll(__ballot(le));
      if (c == 0) { n = 0; break; }
      const int nlo = lo + (c - 1) * stride + 1;
      n = min(stride - 1, lo + n - nlo);
      lo = nlo;
    }
    if (n > 0) {
      const bool le = lane < n && clamp_tok(p.indptr[lo + lane + 1], N) <= seg_lo;
      lo += __popcll(__ballot(le));
    }
    cur_b = __builtin_amdgcn_readfirstlane(lo);
    win = cur_b;
    win_val = clamp_tok(p.indptr[min(win + lane, p.B)], N);
  }
  auto indptr_at = [&](int b) -> int {
    if (b - win > 63) {
      win = b;
      win_val = clamp_tok(p.indptr[min(win + lane, p.B)], N);
    }
    return __builtin_amdgcn_readlane(win_val, b - win);
  };

  int req_lo = 0, req_hi = 0;
  if (cur_b < p.B) {
    req_lo = indptr_at(cur_b);
    req_hi = indptr_at(cur_b + 1);
  }

  // ---- query operand (B of the score MFMA), staged once per workgroup in LDS
  // in operand order: piece c = 64s + l holds, for step s = 2i+e and lane
  // l = (t, g), q[head t][64i + 16g + 8e .. +8] -- the d-order in which lane
  // (t, g) reads its K row.  Heads >= H read the last head and are zeroed.
  auto q_piece_offset = [&](int b, int c) -> int64_t {
    const int s = c >> 6, l = c & 63;
    const int h = min(hg * HEADS + (l & 15), p.H - 1);
    const int d = 64 * (s >> 1) + 16 * (l >> 4) + 8 * (s & 1);
    return ((int64_t)b * p.H + h) * KV_WIDTH + d;
  };
  int qsel = 0;  // which q_lds buffer holds the current query
  auto store_q_piece = [&](int c, u32x4_t v) {
    if (hg * HEADS + ((c & 63) & 15) >= p.H) v = u32x4_t{0u, 0u, 0u, 0u};
    q_lds[qsel][c >> 6][c & 63] = v;
  };

  wait_vm<0>();
  pin(ix0);
  pin(ix1);
  pin(ix2);
  // Prologue: only the first request's query (3 pieces per thread) and the
  // rows of tile 0 are requested before computing starts.  Every workgroup
  // starts at once; had tiles 1 and 2 been requested too, tile 0 would queue
  // behind three tiles' worth of traffic from the whole GPU.
  {
    u32x4_t q0v[3];
    const int b0 = min(cur_b, p.B - 1);
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int c = threadIdx.x + j * THREADS < QPIECES ? threadIdx.x + j * THREADS : threadIdx.x;
      q0v[j] = issue_load_16(p.q + q_piece_offset(b0, c));
    }
    load_rows(ix0, kb0);
    wait_vm<0>();
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      pin(q0v[j]);
      const int c = threadIdx.x + j * THREADS;
      if (c < QPIECES) store_q_piece(c, q0v[j]);
    }
    pin(kb0);
    store_rows(kb0);
  }
  int q_b = cur_b;
  __syncthreads();
  // Then, in the main loop's order ("index of j+1 before rows of j"): index of
  // tile 3, rows of tiles 1 and 2.
  ix0 = load_index(3);
  load_rows(ix1, kb1);
  load_rows(ix2, kb2);
  // Request switch inside the segment: reload the query (compiler-managed
  // loads).  Every wave has passed the barriers of the previous piece, so no
  // one still reads the old query.
  auto load_q = [&](int b) {
    for (int c = threadIdx.x; c < QPIECES; c += THREADS) store_q_piece(c, *reinterpret_cast<const u32x4_t*>(p.q + q_piece_offset(b, c)));
    __syncthreads();
    q_b = b;
  };
  // Next request's query, copied into the idle q_lds buffer one tile ahead
  // of the switch.  Called at a tile's top between the index load and the row
  // loads: the next tile's "at most 10 outstanding" wait then proves the copy
  // landed, since it sits between two operations that wait already covers.
  // Heads >= H get the last head's values (their outputs are never written).
  int pref_b = -1;
  auto maybe_prefetch_q = [&](int k) {
    if (pref_b >= 0 || cur_b + 1 >= p.B) return;
    const int nlo = seg_lo + (k + 1) * TILE;
    const int nhi = min(nlo + TILE, seg_hi);
    if (req_hi < nlo || req_hi >= nhi) return;  // the switch is not in tile k+1
    const int nb = cur_b + 1;
    if (indptr_at(nb + 1) <= req_hi) return;  // next request empty: slow path
    const uint32_t qbase = (uint32_t)(uintptr_t)(
        (__attribute__((address_space(3))) u32x4_t*)&q_lds[qsel ^ 1][0][0]);
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      if (j < 2 || w < 2) {  // 1152 pieces = 2 x 512 + 128
        const int c = THREADS * j + 64 * w + lane;
        issue_lds_dma16(p.q + q_piece_offset(nb, c),
                        __builtin_amdgcn_readfirstlane(qbase + 16 * (THREADS * j + 64 * w)));
      }
    }
    pref_b = nb;
  };
  auto switch_q = [&](int b) {
    if (pref_b == b) {  // every wave's copy has landed (see maybe_prefetch_q)
      __syncthreads();
      qsel ^= 1;
      q_b = b;
    } else {
      load_q(b);
    }
    pref_b = -1;
  };


  // ---- LDS read offsets.  Score operand: lane (t, g) reads chunk 4i + g
  // (bytes 64i + 16g .. +16) of MFMA row t, i.e. tile row tile_row(w, t).
  const int k_off = tile_row(w, t) * ROWB + 16 * g;
  // Transposed value reads.  For P.V step st (tokens 32st..32st+31) lane i
  // of group g supplies row 32st + 4g + i/2 (i/2 < 4, wave 2st's MFMA rows
  // 4g..4g+3) or row 32st + 16 + 4(g^3) + i/2 - 4 (wave 2st+1's rows
  // (4g..4g+3)^12): exactly the tokens whose probabilities this lane holds.
  // Rows of later steps are 32 rows further, an immediate offset.
  const int tr_row0 = (t >> 1) < 4 ? 4 * g + (t >> 1) : 16 + 4 * (g ^ 3) + (t >> 1) - 4;
  const int tr_off = tr_row0 * ROWB + 8 * (t & 1) + 64 * w;
  // first tile-relative token of this lane's four score rows (4g..4g+3 of
  // wave w, XOR 12 on odd waves): a run of 4 consecutive tokens
  const int s_tok0 = 16 * w + 4 * ((w & 1) ? (g ^ 3) : g);

  f32x4_t O[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) O[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;
  float l_w = 0.f;
  i32x2_t vt[4][4];  // value operand of the current tile, read once per tile

  // One piece (the part of a tile that belongs to one request).  When
  // `next` is non-null this is the tile's last piece: after the max exchange
  // (every wave is past its reads of the row tile) the next tile's rows are
  // staged, and the probability exchange barrier publishes them.
  auto run_piece = [&](int tile_lo, int plo, int phi, u32x4_t* next) {
    f32x4_t a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
    const uint8_t* kp = kv_lds + k_off;
#pragma unroll
    for (int i = 0; i < KCHUNKS; ++i) {
      const u32x4_t kv = *reinterpret_cast<const u32x4_t*>(kp + 64 * i);
      a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16x8(kv[0], kv[1]),
                                                   __builtin_bit_cast(bf16x8_t, q_lds[qsel][2 * i][lane]),
                                                   a0, 0, 0, 0);
      a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16x8(kv[2], kv[3]),
                                                   __builtin_bit_cast(bf16x8_t, q_lds[qsel][2 * i + 1][lane]),
                                                   a1, 0, 0, 0);
    }
    float s[4];
    float lmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tok = tile_lo + s_tok0 + r;
      const bool ok = tok >= plo && tok < phi;
      s[r] = ok ? (a0[r] + a1[r]) * p.score_scale : -INFINITY;
      lmax = fmaxf(lmax, s[r]);
    }
    lmax = wave_max_over_groups(lmax);
    if (g == 0) mx_lds[w][t] = lmax;
    __syncthreads();
    if (next) {
      // The next tile's rows were issued before 19 or more younger operations
      // (tile 0: rows of tiles 2 and 3 and an index; later tiles: two tiles'
      // rows and indices), so "at most 19 outstanding" proves they arrived.
      u32x4_t (&nk)[KCHUNKS] = *reinterpret_cast<u32x4_t(*)[KCHUNKS]>(next);
      wait_vm<19>();
      pin(nk);
      store_rows(nk);
    }
    float tmax = mx_lds[0][t];
#pragma unroll
    for (int v = 1; v < NWAVES; ++v) tmax = fmaxf(tmax, mx_lds[v][t]);
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    if (__ballot(alpha != 1.0f)) {
#pragma unroll
      for (int c = 0; c < 4; ++c) O[c] *= alpha;
      l_w *= alpha;
    }
    m_run = m_new;
    float pr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) pr[r] = __builtin_amdgcn_exp2f(s[r] - m_new);
    const uint32_t p01 = pack_bf16x2(pr[0], pr[1]);
    const uint32_t p23 = pack_bf16x2(pr[2], pr[3]);
    l_w += (bf16_bits_to_f32(p01 & 0xFFFFu) + bf16_bits_to_f32(p01 >> 16)) +
           (bf16_bits_to_f32(p23 & 0xFFFFu) + bf16_bits_to_f32(p23 >> 16));
    p_lds[w][lane] = make_uint2(p01, p23);
    __syncthreads();

    bf16x8_t pb[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const uint2 x = p_lds[2 * st][lane];
      const uint2 y = p_lds[2 * st + 1][lane];
      u32x4_t v = {x.x, x.y, y.x, y.y};
      pb[st] = __builtin_bit_cast(bf16x8_t, v);
    }
    // Rows of the tile outside this piece (another request, or past the
    // segment) have probability 0; their value bytes are zeroed as well so
    // that a NaN in another request's rows cannot enter through 0 * NaN.
    const bool mask_v = plo > tile_lo || phi < tile_lo + TILE;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      uint32_t mlo = 0xFFFFFFFFu, mhi = 0xFFFFFFFFu;
      if (mask_v) {
        // bytes jj < 4: tokens 32st + 4g + jj; bytes jj >= 4: 32st + 16 + 4(g^3) + jj - 4
        mlo = run_mask(tile_lo + 32 * st + 4 * g, plo, phi);
        mhi = run_mask(tile_lo + 32 * st + 16 + 4 * (g ^ 3), plo, phi);
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t lo = (uint32_t)vt[st][c].x & mlo;
        const uint32_t hi = (uint32_t)vt[st][c].y & mhi;
        O[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16x8(lo, hi), pb[st], O[c], 0, 0, 0);
      }
    }
  };

  auto finish_piece = [&](bool complete) {
    const float lsum = wave_sum_over_groups(l_w);
    if (g == 0) l_lds[w][t] = lsum;
    __syncthreads();
    float l = 0.f;
#pragma unroll
    for (int v = 0; v < NWAVES; ++v) l += l_lds[v][t];
    if (complete) {
      if (head < p.H) {
        const float inv = p.kv_scale / l;
        uint16_t* op = p.out + ((int64_t)cur_b * p.H + head) * V_WIDTH + 64 * w + 4 * g;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          uint2 v;
          v.x = pack_bf16x2(O[c][0] * inv, O[c][1] * inv);
          v.y = pack_bf16x2(O[c][2] * inv, O[c][3] * inv);
          *reinterpret_cast<uint2*>(op + 16 * c) = v;
        }
      }
    } else {
      const int64_t piece = (int64_t)(seg + cur_b) * p.Hp + head;
      const float inv = 1.0f / l;
      float* op = p.part_o + piece * V_WIDTH + 64 * w + 4 * g;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        *reinterpret_cast<float4*>(op + 16 * c) =
            make_float4(O[c][0] * inv, O[c][1] * inv, O[c][2] * inv, O[c][3] * inv);
      if (w == 0 && g == 0) p.part_lse[piece] = m_run + __builtin_amdgcn_logf(l);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) O[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    l_w = 0.f;
    m_run = -INFINITY;
  };

  // Tile k: its rows are in the LDS tile (published by the previous
  // barrier); `next` holds the rows of tile k+1 in registers (they have
  // arrived) and is staged during the tile's last piece.
  auto process_tile = [&](int k, u32x4_t (&next)[KCHUNKS]) {
    const int tile_lo = seg_lo + k * TILE;
    const int tile_hi = min(tile_lo + TILE, seg_hi);
    {
      const uint8_t* vbase = kv_lds + tr_off;
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          vt[st][c] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (__attribute__((address_space(3))) i32x2_t*)(vbase + 32 * ROWB * st + 16 * c));
    }
    int pos = tile_lo;
    bool staged = false;
    while (pos < tile_hi) {
      while (req_hi <= pos && cur_b < p.B) {
        ++cur_b;
        req_lo = req_hi;
        req_hi = cur_b < p.B ? max(req_lo, indptr_at(cur_b + 1)) : req_lo;
      }
      if (cur_b >= p.B) break;  // malformed kv_indptr: tokens past the last request
      const int plo = pos;
      const int phi = min(tile_hi, req_hi);
      if (q_b != cur_b) switch_q(cur_b);
      const bool last = phi == tile_hi;
      run_piece(tile_lo, plo, phi, last ? &next[0] : nullptr);
      staged |= last;
      if (phi == req_hi || phi == seg_hi) finish_piece(req_lo >= seg_lo && req_hi <= seg_hi);
      pos = phi;
    }
    if (!staged) {  // no piece reached the tile end (malformed kv_indptr): keep the barrier count
      __syncthreads();
      wait_vm<19>();
      pin(next);
      store_rows(next);
      __syncthreads();
    }
  };

  // ---- main loop: a three-slot register ring.  At tile k the rows of tile
  // k+1 wait in registers to be staged into LDS (after arriving), and the
  // rows of tiles k+2 and k+3 are in flight.  Issue order per tile: index of
  // tile k+4, then the rows of tile k+3 once the index of k+3 has arrived --
  // "at most 10 outstanding" (rows of k+2, index of k+4) proves it, and also
  // proves the rows of k+1 arrived.  Tile 0 is peeled: there the index of
  // tile 3 precedes the rows of tiles 1 and 2, so 19 may stay outstanding.
  // Ring slots: rows of tile j live in kb[j % 3]; indices of tile j in ix[j % 3].
  ix1 = load_index(4);
  wait_vm<19>();
  pin(ix0);
  maybe_prefetch_q(0);
  load_rows(ix0, kb0);
  process_tile(0, kb1);
  for (int k = 0; k < ntiles; k += 3) {
    if (k > 0) {
      ix1 = load_index(k + 4);
      wait_vm<10>();
      pin(ix0);
      pin(kb1);
      maybe_prefetch_q(k);
      load_rows(ix0, kb0);
      process_tile(k, kb1);
    }
    if (k + 1 >= ntiles) break;
    ix2 = load_index(k + 5);
    wait_vm<10>();
    pin(ix1);
    pin(kb2);
    maybe_prefetch_q(k + 1);
    load_rows(ix1, kb1);
    process_tile(k + 1, kb2);
    if (k + 2 >= ntiles) break;
    ix0 = load_index(k + 6);
    wait_vm<10>();
    pin(ix2);
    pin(kb0);
    maybe_prefetch_q(k + 2);
    load_rows(ix2, kb2);
    process_tile(k + 2, kb0);
  }
  wait_vm<0>();  // retire prefetches issued past the last tile
}

// One wave per (request, head): merges the partials of a request that spans
// several segments.  out = scale * sum_s w_s o_s / sum_s w_s with
// w_s = 2^(lse_s - max lse).  Requests with no tokens get zeros; requests
// inside one segment were written by the split kernel.  The log-sum-exps of
// up to 64 pieces are loaded in one wave-wide step and the partial outputs
// four pieces at a time, so a request costs one or two memory latencies, not
// one per piece.
__global__ __launch_bounds__(256) void mla_combine_kernel(const CombineParams p) {
  const int b = blockIdx.x;
  const int head = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (head >= p.H) return;
  const int N = p.total_tokens;
  const int lo = clamp_tok(p.indptr[b], N);
  const int hi = max(lo, clamp_tok(p.indptr[b + 1], N));
  uint16_t* op = p.out + ((int64_t)b * p.H + head) * V_WIDTH + 8 * lane;
  if (hi <= lo) {
    *reinterpret_cast<uint4*>(op) = make_uint4(0u, 0u, 0u, 0u);
    return;
  }
  const int s0 = lo / p.seg_len;
  const int s1 = (hi - 1) / p.seg_len;
  if (s0 == s1) return;
  const int np = s1 - s0 + 1;
  const float* lse = p.part_lse + (int64_t)(s0 + b) * p.Hp + head;  // piece i at lse[i * Hp]
  float M = -INFINITY;
  for (int i = lane; i < np; i += 64) M = fmaxf(M, lse[(int64_t)i * p.Hp]);
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  const float* po = p.part_o + ((int64_t)(s0 + b) * p.Hp + head) * V_WIDTH + 8 * lane;
  const int64_t pstride = (int64_t)p.Hp * V_WIDTH;  // floats between consecutive pieces
  for (int base = 0; base < np; base += 64) {
    const int cnt = min(64, np - base);
    const float wl = lane < cnt ? __builtin_amdgcn_exp2f(lse[(int64_t)(base + lane) * p.Hp] - M) : 0.f;
    int i = 0;
    for (; i + 4 <= cnt; i += 4) {
      float4 x[4], y[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float4* q = reinterpret_cast<const float4*>(po + (int64_t)(base + i + u) * pstride);
        x[u] = q[0];
        y[u] = q[1];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float wgt =
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), i + u));
        acc[0] += wgt * x[u].x; acc[1] += wgt * x[u].y; acc[2] += wgt * x[u].z; acc[3] += wgt * x[u].w;
        acc[4] += wgt * y[u].x; acc[5] += wgt * y[u].y; acc[6] += wgt * y[u].z; acc[7] += wgt * y[u].w;
        den += wgt;
      }
    }
    for (; i < cnt; ++i) {
      const float4* q = reinterpret_cast<const float4*>(po + (int64_t)(base + i) * pstride);
      const float4 x = q[0], y = q[1];
      const float wgt = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), i));
      acc[0] += wgt * x.x; acc[1] += wgt * x.y; acc[2] += wgt * x.z; acc[3] += wgt * x.w;
      acc[4] += wgt * y.x; acc[5] += wgt * y.y; acc[6] += wgt * y.z; acc[7] += wgt * y.w;
      den += wgt;
    }
  }
  const float inv = p.kv_scale / den;
  uint4 v;
  v.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  v.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
  v.z = pack_bf16x2(acc[4] * inv, acc[5] * inv);
  v.w = pack_bf16x2(acc[6] * inv, acc[7] * inv);
  *reinterpret_cast<uint4*>(op) = v;
}

}  // namespace

DecodePlan plan_mla_decode(int32_t batch, int32_t num_heads, int64_t total_tokens, int num_cus) {
  DecodePlan pl{};
  pl.HG = (num_heads + HEADS - 1) / HEADS;
  pl.Hp = pl.HG * HEADS;
  if (total_tokens <= 0) return pl;
  // one 8-wave workgroup per compute unit in flight; head groups of a segment
  // are separate workgroups that share the segment's rows through L2
  int64_t nseg_target = num_cus / pl.HG;
  if (nseg_target < 1) nseg_target = 1;
  // Segments need no alignment (tiles are counted from each segment's start),
  // so the token stream is cut into exactly nseg_target pieces when it can be.
  const int64_t seg = (total_tokens + nseg_target - 1) / nseg_target;
  pl.seg_len = (int32_t)seg;
  pl.nseg = (int32_t)((total_tokens + seg - 1) / seg);
  pl.items = pl.nseg * pl.HG;
  if (pl.HG > 1) {
    pl.xcd_per = (pl.items + 7) / 8;
    pl.grid = 8 * pl.xcd_per;
  } else {
    pl.xcd_per = pl.items;
    pl.grid = pl.items;
  }
  const size_t npieces = (size_t)pl.nseg + (size_t)batch;
  const size_t o_bytes = npieces * pl.Hp * V_WIDTH * sizeof(float);
  const size_t lse_bytes = npieces * pl.Hp * sizeof(float);
  pl.lse_offset = (o_bytes + 255) / 256 * 256;
  pl.workspace_bytes = pl.lse_offset + (lse_bytes + 255) / 256 * 256;
  return pl;
}

hipError_t launch_mla_decode(const uint16_t* q, const uint8_t* kv_pool, int64_t num_slots,
                             const int32_t* kv_indptr, const int32_t* kv_indices,
                             int64_t total_tokens, int32_t batch, int32_t num_heads, float scale,
                             float sm_scale, uint16_t* out, void* workspace, const DecodePlan& pl,
                             hipStream_t stream) {
  float* part_o = reinterpret_cast<float*>(workspace);
  float* part_lse = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + pl.lse_offset);
  if (total_tokens > 0) {
    SplitParams sp;
    sp.q = q;
    sp.pool = kv_pool;
    sp.indptr = kv_indptr;
    sp.indices = kv_indices;
    sp.out = out;
    sp.part_o = part_o;
    sp.part_lse = part_lse;
    sp.max_slot = (uint32_t)(num_slots - 1);
    sp.total_tokens = (int32_t)total_tokens;
    sp.B = batch;
    sp.H = num_heads;
    sp.HG = pl.HG;
    sp.Hp = pl.Hp;
    sp.seg_len = pl.seg_len;
    sp.items = pl.items;
    sp.xcd_per = pl.xcd_per;
    sp.score_scale = (float)((double)sm_scale * (double)scale * 1.4426950408889634);
    sp.kv_scale = scale;
    hipLaunchKernelGGL(mla_split_kernel, dim3(pl.grid), dim3(THREADS), 0, stream, sp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  CombineParams cp;
  cp.indptr = kv_indptr;
  cp.part_o = part_o;
  cp.part_lse = part_lse;
  cp.out = out;
  cp.total_tokens = (int32_t)total_tokens;
  cp.B = batch;
  cp.H = num_heads;
  cp.Hp = pl.Hp;
  cp.seg_len = pl.seg_len > 0 ? pl.seg_len : 1;
  cp.kv_scale = scale;
  hipLaunchKernelGGL(mla_combine_kernel, dim3(batch, (num_heads + 3) / 4), dim3(256), 0, stream, cp);
  return hipGetLastError();
}

}  // namespace fp8mla
