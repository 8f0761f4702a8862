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
// Work decomposition.  Every request's token range is cut into tiles of 128
// tokens counted from the request's start (its last tile may be partial), so
// no tile mixes two requests.  The concatenated list of all requests' tiles
// is cut into equal segments, one per compute unit and group of 16 heads:
// segments are balanced by tiles, not by request, so long and short requests
// cost the same per token.  For every request it touches a workgroup writes
// either the final output (request entirely inside the segment) or a partial
// (o normalised, fp16, and its log2-sum-exp) that the combine kernel merges.
//
// Inside a workgroup (8 waves, 16 heads), per tile:
//  * the tile's 128 rows are copied global -> LDS by the waves themselves
//    (global_load_lds, 16 bytes per lane) two tiles ahead of use, into one of
//    two LDS slots; no registers are held by rows in flight;
//  * wave w computes the scores of tokens [16w, 16w+16): S^T = K q^T with
//    MFMA 16x16x32 bf16 (M = 16 tokens, N = 16 heads, K = 576 in 18 steps),
//    K read from LDS and converted FP8 -> bf16 right before the MFMA, q held
//    in registers for as long as the request lasts;
//  * the softmax is exchanged through LDS (wave maxima, then bf16
//    probabilities) so that all waves share one running maximum per head;
//  * wave w owns output columns [64w, 64w+64) of O^T = V^T P^T (MFMA
//    16x16x32 bf16, M = 16 columns, N = 16 heads, K = 32 tokens), reading the
//    transposed FP8 value operand with ds_read_b64_tr_b8: no cross-wave
//    reduction of O.
// KV bytes move from HBM once per head group; each value byte is converted
// once per wave that consumes it.
#include "device_common.h"
#include "launch.h"

#include <math.h>

namespace fp8mla {
namespace {

constexpr int NWAVES = 8;
constexpr int THREADS = 64 * NWAVES;              // 512
constexpr int TILE = 16 * NWAVES;                 // tokens per tile: 16 per wave
constexpr int TILE_SHIFT = 7;                     // log2(TILE)
constexpr int HEADS = 16;                         // heads per workgroup
constexpr int ROW_SLOTS = KV_CHUNKS + 1;          // 16-byte LDS slots per row: 36 + 1 pad (odd)
constexpr int ROWB = 16 * ROW_SLOTS;              // 592 LDS bytes per row
constexpr int TILE_BYTES = TILE * ROWB;           // 75776
constexpr int KSTEPS = KV_WIDTH / 64;             // 16-byte K reads per lane per tile; query steps / 2
constexpr int QSTEPS = 2 * KSTEPS;                // 18 MFMA steps of 32 dims over 576
constexpr int DMA_OPS = (16 * ROW_SLOTS + 63) / 64;  // LDS-copy ops per wave per tile: 10
static_assert(TILE == 1 << TILE_SHIFT, "tile size");
constexpr int TILE_W = 4;   // segment balancing: weight of a tile
constexpr int START_W = 2;  // extra weight of a request's first tile

struct SplitParams {
  const uint16_t* q;
  const uint8_t* pool;
  const int32_t* indptr;
  const int32_t* indices;
  uint16_t* out;
  uint16_t* part_o;  // fp16 bits
  float* part_lse;
  int2* req_pieces;  // per request: (segment of its first piece, number of pieces)
  uint32_t max_slot;
  int32_t total_tokens;
  int32_t B;
  int32_t H;
  int32_t HG;
  int32_t Hp;
  int32_t nseg;     // segments the tile list is cut into
  int32_t items;    // nseg * HG
  int32_t xcd_per;
  float score_scale;  // sm_scale * scale * log2(e): scores in the base-2 domain
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

// ---- request tiles.  Request b covers tokens [lo_b, hi_b) with
// lo_b = clamp(kv_indptr[b], 0, N) and hi_b = max(lo_b, clamp(kv_indptr[b+1],
// 0, N)), and has ceil((hi_b - lo_b) / 128) tiles.
__device__ __forceinline__ int request_tiles(const int32_t* indptr, int b, int B, int N) {
  if (b >= B) return 0;
  const int lo = clamp_tok(indptr[b], N);
  const int hi = max(lo, clamp_tok(indptr[b + 1], N));
  return (hi - lo + TILE - 1) >> TILE_SHIFT;
}

__device__ __forceinline__ int wave_sum_i32(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

__device__ __forceinline__ int wave_inclusive_scan(int x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

// Merge of the np partial results (pieces s0 + b .. s0 + np - 1 + b) of
// request b for one head, by one wave: out = scale * sum_s w_s o_s / sum_s
// w_s with w_s = 2^(lse_s - max lse).  Pieces are taken eight at a time with
// all their loads issued together (one memory latency per eight pieces) and
// folded in with a running maximum.  Lane l produces output columns
// 8l .. 8l+7.
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;

// Partial outputs are stored as fp16 (round to nearest even), in E4M3 units
// (before the per-tensor scale): every partial is a convex combination of
// E4M3 values, |o| <= 448, so fp16 cannot overflow, and its 11-bit
// significand is finer than the bf16 the merged output is rounded to.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  const f16x2_t v = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float f16_lo(uint32_t w) { return (float)__builtin_bit_cast(f16x2_t, w).x; }
__device__ __forceinline__ float f16_hi(uint32_t w) { return (float)__builtin_bit_cast(f16x2_t, w).y; }

__device__ __forceinline__ void merge_pieces(const uint16_t* part_o, const float* part_lse, int Hp,
                                             int b, int s0, int np, int head, float kv_scale,
                                             uint16_t* op, int lane) {
  const float* lse = part_lse + (int64_t)(s0 + b) * Hp + head;  // piece i at lse[i * Hp]
  const uint16_t* po = part_o + ((int64_t)(s0 + b) * Hp + head) * V_WIDTH + 8 * lane;
  const int64_t pstride = (int64_t)Hp * V_WIDTH;  // elements between consecutive pieces
  float M = -INFINITY, den = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int base = 0; base < np; base += 8) {
    const int cnt = min(8, np - base);
    const float lv = lane < cnt ? lse[(int64_t)(base + lane) * Hp] : -INFINITY;
    uint4 x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)  // u >= cnt re-reads the last piece (in bounds, unused)
      x[u] = *reinterpret_cast<const uint4*>(po + (int64_t)(base + min(u, cnt - 1)) * pstride);
    float cm = lv;
#pragma unroll
    for (int off = 1; off < 8; off <<= 1) cm = fmaxf(cm, __shfl_xor(cm, off));
    const float m_new = fmaxf(M, __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                                     __builtin_bit_cast(int, cm))));
    const float r = __builtin_amdgcn_exp2f(M - m_new);  // 0 on the first chunk
    den *= r;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= r;
    M = m_new;
    const float wl = lane < cnt ? __builtin_amdgcn_exp2f(lv - M) : 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (u < cnt) {
        const float wgt = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), u));
        acc[0] += wgt * f16_lo(x[u].x); acc[1] += wgt * f16_hi(x[u].x);
        acc[2] += wgt * f16_lo(x[u].y); acc[3] += wgt * f16_hi(x[u].y);
        acc[4] += wgt * f16_lo(x[u].z); acc[5] += wgt * f16_hi(x[u].z);
        acc[6] += wgt * f16_lo(x[u].w); acc[7] += wgt * f16_hi(x[u].w);
        den += wgt;
      }
    }
  }
  const float inv = kv_scale / den;
  uint4 v;
  v.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  v.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
  v.z = pack_bf16x2(acc[4] * inv, acc[5] * inv);
  v.w = pack_bf16x2(acc[6] * inv, acc[7] * inv);
  *reinterpret_cast<uint4*>(op + 8 * lane) = v;
}

// ---- explicitly pipelined loads.  Index, query and row copies are issued as
// inline assembly and waited for with an explicit s_waitcnt vmcnt(N): left to
// itself the compiler sinks prefetches down to their first use or drains
// every load at a barrier, which removes the overlap the pipeline exists
// for.  Loads (register and LDS-destination alike) complete in issue order,
// so "at most N outstanding" proves every load older than the N youngest
// done; stores, which the compiler may interleave, only make such a wait
// stricter.  After a wait, pin() makes the compiler treat the registers as
// redefined there, so no use of the data can be scheduled above the wait.
__device__ __forceinline__ int32_t issue_load_i32(const int32_t* p) {
  int32_t v;
  asm volatile("global_load_dword %0, %1, off" : "=v"(v) : "v"(p));
  return v;
}

// Global -> LDS copy of 16 bytes per lane: lane l's bytes land at LDS byte
// address lds_base + 16*l (lds_base wave-uniform, passed in M0); lanes
// outside exec write nothing.  The caller waits with vmcnt.  M0 is not
// otherwise used by these kernels.
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

// Wait until at most n vector-memory operations are outstanding (n is
// wave-uniform and one of the counts the pipeline produces; any other value
// waits for everything).
__device__ __forceinline__ void wait_vm_upto(int n) {
  switch (n) {
    case 1: wait_vm<1>(); break;
    case 10: wait_vm<10>(); break;
    case 11: wait_vm<11>(); break;
    default: wait_vm<0>(); break;
  }
}

__device__ __forceinline__ void pin(int32_t& x) { asm volatile("" : "+v"(x)); }

// Token row (tile-relative) held by MFMA row m of wave w.  Odd waves use
// row m ^ 12 so that the transposed LDS reads of two consecutive waves'
// rows fall in distinct banks.
__device__ __forceinline__ int tile_row(int w, int m) { return 16 * w + ((w & 1) ? (m ^ 12) : m); }

// Walks the tiles of consecutive requests: request b, tile j of its nt
// tiles, request range [lo, hi).  Requests without tokens are skipped.  The
// kv_indptr values come from a 64-entry window held one entry per lane.
struct TileCursor {
  int b, j, nt, lo, hi;
  int win, win_val;
  __device__ __forceinline__ int tile_lo() const { return lo + (j << TILE_SHIFT); }
  __device__ __forceinline__ int tile_hi() const { return min(tile_lo() + TILE, hi); }
};

__global__ __launch_bounds__(THREADS) void mla_split_kernel(const SplitParams p) {
  // Two row tiles (the one being computed and the next one landing) and the
  // softmax exchange.
  __shared__ __attribute__((aligned(16))) uint8_t kv_lds[2 * TILE_BYTES];
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
  const int head = hg * HEADS + t;  // head whose scores / outputs this lane carries

  // ---- this segment's tiles.  Tiles are weighted by their cost: TILE_W per
  // tile and START_W more for the first tile of a request (the query switch
  // and the extra output).  Request b's tile j sits at weighted position
  // x = P_b + START_W + TILE_W * j, P_b being the total weight of the
  // requests before b; segment s takes the tiles with x in
  // [ceil(s W / nseg), ceil((s+1) W / nseg)), W the total weight, so tile x
  // belongs to segment floor(x nseg / W).  Found with two wave-wide scans
  // over the requests, 64 per step: the global index t0 of the first tile,
  // its request b0 and tile j0, and the number of tiles.
  // (Weights fit in int: W <= 4 * (N / 128 + B) + 2 * B.)
  int W = 0;
  for (int c = 0; c < p.B; c += 64) {
    const int nt = request_tiles(p.indptr, c + lane, p.B, N);
    W += wave_sum_i32(nt > 0 ? TILE_W * nt + START_W : 0);
    // requests without tokens: zero outputs, written by the first segment
    uint64_t empty = seg == 0 ? __ballot(c + lane < p.B && nt == 0) : 0ull;
    while (empty) {
      const int b = c + __builtin_ctzll(empty);
      empty &= empty - 1;
      if (hg == 0 && threadIdx.x == 0 && p.req_pieces) p.req_pieces[b] = make_int2(0, 0);
      for (int i = threadIdx.x; i < HEADS * 64; i += THREADS) {
        const int h = hg * HEADS + (i >> 6);
        if (h < p.H)
          *reinterpret_cast<uint4*>(p.out + ((int64_t)b * p.H + h) * V_WIDTH + 8 * (i & 63)) =
              make_uint4(0u, 0u, 0u, 0u);
      }
    }
  }
  // Consecutive tile positions are at most TILE_W + START_W apart, so with
  // segments at least that wide every segment holds a tile and the pieces of
  // a request are consecutive segments; later workgroups stay idle.
  const int nseg = min(p.nseg, W / (TILE_W + START_W));
  if (seg >= nseg) return;
  const int x_lo = (int)(((int64_t)seg * W + nseg - 1) / nseg);
  const int x_hi = (int)(((int64_t)(seg + 1) * W + nseg - 1) / nseg);
  auto segment_of = [&](int x) -> int { return (int)((int64_t)x * nseg / W); };
  // global index t0 of the first tile at or after x_lo (its request b0, tile
  // j0, weight P0 before b0) and t1 of the first at or after x_hi
  int t0 = -1, t1 = -1, b0 = 0, j0 = 0, P0 = 0;
  {
    int wcarry = 0, tcarry = 0;
    for (int c = 0; c < p.B && t1 < 0; c += 64) {
      const int nt = request_tiles(p.indptr, c + lane, p.B, N);
      const int w = nt > 0 ? TILE_W * nt + START_W : 0;
      const int Pb = wcarry + wave_inclusive_scan(w, lane) - w;
      const int TB = tcarry + wave_inclusive_scan(nt, lane) - nt;
      const int last_x = Pb + START_W + TILE_W * (nt - 1);
      auto first_at = [&](int X, int& t, bool keep) {
        const uint64_t hit = __ballot(nt > 0 && last_x >= X);
        if (t >= 0 || !hit) return;
        const int l = __builtin_ctzll(hit);
        const int pb = __builtin_amdgcn_readlane(Pb, l);
        const int rel = X - pb - START_W;
        const int j = rel <= 0 ? 0 : (rel + TILE_W - 1) / TILE_W;
        t = __builtin_amdgcn_readlane(TB, l) + j;
        if (keep) {
          b0 = c + l;
          j0 = j;
          P0 = pb;
        }
      };
      first_at(x_lo, t0, true);
      first_at(x_hi, t1, false);
      wcarry += wave_sum_i32(w);
      tcarry += wave_sum_i32(nt);
      if (c + 64 >= p.B && t1 < 0) t1 = tcarry;  // past the last tile
    }
  }
  if (t0 < 0) return;
  const int ntiles = t1 - t0;
  if (ntiles <= 0) return;
  auto load_window = [&](TileCursor& c, int b) {
    c.win = b;
    c.win_val = clamp_tok(p.indptr[min(b + lane, p.B)], N);
  };
  // (every field assigned exactly once on every path, so that the cursors
  // stay in registers)
  auto set_request = [&](TileCursor& c, int b) {
    const bool valid = b < p.B;  // past the last request: an empty cursor
    if (valid && b + 1 - c.win > 63) load_window(c, b);
    const int lo = __builtin_amdgcn_readlane(c.win_val, valid ? b - c.win : 0);
    const int hi = max(lo, __builtin_amdgcn_readlane(c.win_val, valid ? b + 1 - c.win : 0));
    c.b = b;
    c.lo = valid ? lo : 0;
    c.hi = valid ? hi : 0;
    c.nt = valid ? (hi - lo + TILE - 1) >> TILE_SHIFT : 0;
  };
  auto advance = [&](TileCursor& c) {
    if (++c.j < c.nt) return;
    c.j = 0;
    do {
      set_request(c, c.b + 1);
    } while (c.nt == 0 && c.b < p.B);
  };
  TileCursor cc;  // tile being computed
  load_window(cc, b0);
  set_request(cc, b0);
  cc.j = j0;
  TileCursor lc = cc;  // next tile whose index is loaded

  // ---- row tiles.  Tile k of the segment goes to LDS slot k & 1 by
  // global->LDS copies, two tiles ahead of use.  Token r of the tile is LDS
  // row r (592 bytes: the 576-byte row and a 16-byte pad).  Wave w copies
  // rows 16w..16w+15, a block of 16 x 37 consecutive 16-byte LDS slots: op j
  // fills slots 64j..64j+63 of it, lane l taking slot P = 64j + l, i.e. row
  // P / 37, chunk P % 37; pad slots (chunk 36) get a copy of chunk 35 and the
  // lanes past the block in the last op are masked off.  Each op thus reads
  // whole rows back to back, the pattern that gathers random 576-byte rows
  // fastest.  Lanes r < 16 (and their copies at r + 16k) hold the slot id of
  // row r, which every lane fetches with a cross-lane permute.  Tokens past
  // the tile's request read the tile's first row (a cache hit of the same
  // request); their scores are masked out.
  auto opaque_lane = [&]() -> int {  // recomputed per use, not kept across the loop
    int l = lane;
    asm volatile("" : "+v"(l));
    return l;
  };
  // index of the load cursor's tile, then advance it (past the segment's
  // last tile the load reads entry 0 and is never used)
  auto load_next_index = [&]() -> int32_t {
    const int tlo = lc.tile_lo();
    const int tok = tlo + 16 * w + t;
    const int32_t* a = lc.nt > 0 ? p.indices + (tok < lc.tile_hi() ? tok : tlo) : p.indices;
    const int32_t v = issue_load_i32(a);
    advance(lc);
    return v;
  };
  const uint32_t lds_tiles = (uint32_t)(uintptr_t)(
      (__attribute__((address_space(3))) uint8_t*)&kv_lds[0]);
  auto issue_tile = [&](int k, int32_t idx) {
    const uint32_t base =
        __builtin_amdgcn_readfirstlane(lds_tiles + (uint32_t)((k & 1) * TILE_BYTES + 16 * w * ROWB));
    const int ln = opaque_lane();
#pragma unroll
    for (int j = 0; j < DMA_OPS; ++j) {
      const int P = 64 * j + ln;
      const int r = P / ROW_SLOTS;
      const int c = min(P - r * ROW_SLOTS, KV_CHUNKS - 1);
      const uint32_t s = (uint32_t)__shfl(idx, r & 15);
      const uint8_t* a = p.pool + (uint64_t)(s < p.max_slot ? s : p.max_slot) * KV_WIDTH + 16 * c;
      if (j < DMA_OPS - 1 || P < 16 * ROW_SLOTS) issue_lds_dma16(a, base + 1024 * j);
    }
  };

  // ---- query operand (B of the score MFMA), held in registers: for step
  // s = 2i + e lane (t, g) holds q[head t][64i + 16g + 8e .. +8], the d-order
  // in which it reads its K row.  A request's query is copied once per
  // workgroup into 18 KB of an LDS row slot (3 copy ops per wave; piece
  // c = 64s + l holds lane l's operand for step s) and every wave reads its
  // operand from there: one 18 KB copy through the memory pipeline instead of
  // one per wave.  Heads >= H copy the last head and are zeroed.
  constexpr int QCOPY_OPS = 3;
  constexpr int QCOPY_BYTES = QSTEPS * 64 * 16;  // 18432: rows 0..31 of a slot
  static_assert(QCOPY_BYTES <= 32 * ROWB, "query copy must fit in waves 0-1's rows");
  auto issue_query_copy = [&](int b, uint32_t lds_base) {
#pragma unroll
    for (int j = 0; j < QCOPY_OPS; ++j) {
      // ops 0 and 1: pieces 128w + 64j + l; op 2: pieces 1024 + 64(w & 1) + l
      // (waves of equal parity copy the same bytes to the same place)
      const int c0 = j < 2 ? 128 * w + 64 * j : 1024 + 64 * (w & 1);
      const int c = c0 + opaque_lane();
      const int s = c >> 6, l = c & 63;
      const int h = min(hg * HEADS + (l & 15), p.H - 1);
      const int d = 64 * (s >> 1) + 16 * (l >> 4) + 8 * (s & 1);
      issue_lds_dma16(p.q + ((int64_t)b * p.H + h) * KV_WIDTH + d,
                      __builtin_amdgcn_readfirstlane(lds_base + 16 * c0));
    }
  };
  bf16x8_t qr[QSTEPS];
  auto read_query = [&](const uint8_t* lds_q) {
    const u32x4_t* qs = reinterpret_cast<const u32x4_t*>(lds_q);
#pragma unroll
    for (int s = 0; s < QSTEPS; ++s) qr[s] = __builtin_bit_cast(bf16x8_t, qs[64 * s + lane]);
    if (head >= p.H) {
#pragma unroll
      for (int s = 0; s < QSTEPS; ++s) qr[s] = bf16x8_t{};
    }
  };

  // Prologue.  The first request's query goes through LDS slot 1 (free until
  // tile 1 is requested).  Issue order: indices of tiles 0 and 1, the query,
  // rows of tile 0, index of tile 2; once every wave has read the query, rows
  // of tile 1.
  int32_t ixE = load_next_index();  // even tiles k: holds the index of tile k + 2
  int32_t ixO = load_next_index();  // odd tiles
  issue_query_copy(cc.b, lds_tiles + TILE_BYTES);
  wait_vm<QCOPY_OPS>();  // indices of tiles 0 and 1 landed
  pin(ixE);
  pin(ixO);
  issue_tile(0, ixE);
  ixE = load_next_index();
  wait_vm<1 + DMA_OPS>();  // query landed (younger: rows of tile 0, index of tile 2)
  __syncthreads();
  read_query(kv_lds + TILE_BYTES);
  __syncthreads();  // every wave holds its query: slot 1 may be refilled
  if (ntiles > 1) issue_tile(1, ixO);
  wait_vm_upto(ntiles > 1 ? 1 + DMA_OPS : 1);  // rows of tile 0 landed
  __syncthreads();

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
  bool whole_request = j0 == 0;  // the current request's first tile is in this segment
  int P_cur = P0;                 // weight of the requests before the current one
  // Pieces of a request: the segments its tiles [first, first + nt) fall in.
  // Recorded for the combine by the workgroup holding the request's first
  // tile (head group 0).
  auto record_pieces = [&]() {
    if (hg == 0 && threadIdx.x == 0) {
      const int s0 = segment_of(P_cur + START_W);
      const int s1 = segment_of(P_cur + START_W + TILE_W * (cc.nt - 1));
      p.req_pieces[cc.b] = make_int2(s0, s1 - s0 + 1);
    }
  };
  if (whole_request) record_pieces();

  auto finish_request = [&](bool complete) {
    const float lsum = wave_sum_over_groups(l_w);
    if (g == 0) l_lds[w][t] = lsum;
    __syncthreads();
    float l = 0.f;
#pragma unroll
    for (int v = 0; v < NWAVES; ++v) l += l_lds[v][t];
    if (complete) {
      if (head < p.H) {
        const float inv = p.kv_scale / l;
        uint16_t* op = p.out + ((int64_t)cc.b * p.H + head) * V_WIDTH + 64 * w + 4 * g;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          uint2 v;
          v.x = pack_bf16x2(O[c][0] * inv, O[c][1] * inv);
          v.y = pack_bf16x2(O[c][2] * inv, O[c][3] * inv);
          *reinterpret_cast<uint2*>(op + 16 * c) = v;
        }
      }
    } else {
      const int64_t piece = (int64_t)(seg + cc.b) * p.Hp + head;
      const float inv = 1.0f / l;
      uint16_t* op = p.part_o + piece * V_WIDTH + 64 * w + 4 * g;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        *reinterpret_cast<uint2*>(op + 16 * c) =
            make_uint2(pack_f16x2(O[c][0] * inv, O[c][1] * inv), pack_f16x2(O[c][2] * inv, O[c][3] * inv));
      if (w == 0 && g == 0) p.part_lse[piece] = m_run + __builtin_amdgcn_logf(l);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) O[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    l_w = 0.f;
    m_run = -INFINITY;
  };

  // Tile k: its rows are in slot k & 1 (published by the previous barrier);
  // ix_cur holds the index of tile k+2 and ix_next receives that of tile k+3.
  //   scores -> [barrier: maxima] -> loads for later tiles -> probabilities
  //   -> wait for tile k+1's rows -> [barrier: probabilities, tile k+1]
  //   -> P.V -> (request end: output)
  // After the first barrier every wave is past its reads of slot k & 1, so
  // the rows of tile k+2 may be copied into it.
  auto process_tile = [&](int k, int32_t& ix_cur, int32_t& ix_next) {
    const int tile_lo = cc.tile_lo();
    const int tile_hi = cc.tile_hi();
    const bool last_of_request = cc.j + 1 == cc.nt;
    const uint8_t* slot = kv_lds + (k & 1) * TILE_BYTES;

    f32x4_t a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
    const uint8_t* kp = slot + k_off;
#pragma unroll
    for (int i = 0; i < KSTEPS; ++i) {
      const u32x4_t kv = *reinterpret_cast<const u32x4_t*>(kp + 64 * i);
      a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16x8(kv[0], kv[1]), qr[2 * i], a0, 0, 0, 0);
      a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16x8(kv[2], kv[3]), qr[2 * i + 1], a1, 0, 0, 0);
    }
    // value operand, read before the barrier after which the slot is refilled
    i32x2_t vt[4][4];
    {
      const uint8_t* vbase = slot + tr_off;
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          vt[st][c] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (__attribute__((address_space(3))) i32x2_t*)(vbase + 32 * ROWB * st + 16 * c));
    }
    float s[4];
    float lmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool ok = tile_lo + s_tok0 + r < tile_hi;
      s[r] = ok ? (a0[r] + a1[r]) * p.score_scale : -INFINITY;
      lmax = fmaxf(lmax, s[r]);
    }
    lmax = wave_max_over_groups(lmax);
    if (g == 0) mx_lds[w][t] = lmax;
    __syncthreads();

    // Loads for later tiles: index of tile k+3, rows of tile k+2 into this
    // slot.  The index of tile k+2 was issued before the rows of tile k+1, so
    // "at most DMA_OPS outstanding" proves it arrived without waiting for
    // those rows.  When tile k+1 starts a new request, its query is copied
    // into rows 0..31 of this slot first, and waves 0 and 1 (the owners of
    // those rows) copy their rows of tile k+2 only after every wave has read
    // the query (after the next barrier).
    wait_vm_upto(k + 1 < ntiles ? DMA_OPS : 0);
    pin(ix_cur);
    ix_next = load_next_index();
    const bool new_q = last_of_request && k + 1 < ntiles;
    const bool rows_now = k + 2 < ntiles && (!new_q || w >= 2);
    TileCursor nc = cc;
    if (new_q) {
      advance(nc);
      issue_query_copy(nc.b, lds_tiles + (uint32_t)((k & 1) * TILE_BYTES));
    }
    if (rows_now) issue_tile(k + 2, ix_cur);

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
    // rows of tile k+1 (and a new query) landed; younger: index of k+3 unless
    // a query was copied after it, and rows of k+2 if issued
    if (k + 1 < ntiles) wait_vm_upto((new_q ? 0 : 1) + (rows_now ? DMA_OPS : 0));
    __syncthreads();
    if (new_q) {
      read_query(slot);
      __syncthreads();  // every wave holds the new query: rows 0..31 may be refilled
      if (w < 2 && k + 2 < ntiles) issue_tile(k + 2, ix_cur);
    }

    bf16x8_t pb[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const uint2 x = p_lds[2 * st][lane];
      const uint2 y = p_lds[2 * st + 1][lane];
      u32x4_t v = {x.x, x.y, y.x, y.y};
      pb[st] = __builtin_bit_cast(bf16x8_t, v);
    }
    // Rows past the request's end in a partial tile are copies of the tile's
    // first row with probability 0, so their value bytes need no masking.
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        O[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            e4m3x8_to_bf16x8((uint32_t)vt[st][c].x, (uint32_t)vt[st][c].y), pb[st], O[c], 0, 0, 0);

    if (last_of_request || k + 1 == ntiles) finish_request(whole_request && last_of_request);
    if (new_q) {
      P_cur += TILE_W * cc.nt + START_W;
      cc = nc;
      whole_request = true;
      record_pieces();
    } else {
      advance(cc);
    }
  };

  // ---- main loop, unrolled by two so that each index register keeps one
  // role: at even tiles ixE holds the index of tile k+2 and ixO receives
  // that of tile k+3; at odd tiles the other way round.
  for (int k = 0; k < ntiles; k += 2) {
    process_tile(k, ixE, ixO);
    if (k + 1 >= ntiles) break;
    process_tile(k + 1, ixO, ixE);
  }
  wait_vm<0>();  // retire index loads issued past the last tile
}

struct CombineParams {
  const int2* req_pieces;
  const uint16_t* part_o;
  const float* part_lse;
  uint16_t* out;
  int32_t H;
  int32_t Hp;
  float kv_scale;
};

// One wave per (request, head): merges the pieces of a request that spans
// several segments.  Requests without tokens and requests inside one segment
// were written by the split kernel.
__global__ __launch_bounds__(256) void mla_combine_kernel(const CombineParams p) {
  const int b = blockIdx.x;
  const int head = blockIdx.y * 4 + (threadIdx.x >> 6);
  if (head >= p.H) return;
  const int2 rp = p.req_pieces[b];
  if (rp.y <= 1) return;
  merge_pieces(p.part_o, p.part_lse, p.Hp, b, rp.x, rp.y, head, p.kv_scale,
               p.out + ((int64_t)b * p.H + head) * V_WIDTH, threadIdx.x & 63);
}

}  // namespace

DecodePlan plan_mla_decode(int32_t batch, int32_t num_heads, int64_t total_tokens, int num_cus) {
  DecodePlan pl{};
  pl.HG = (num_heads + HEADS - 1) / HEADS;
  pl.Hp = pl.HG * HEADS;
  // One 8-wave workgroup per compute unit in flight; head groups of a
  // segment are separate workgroups that share the segment's rows through
  // L2.  The tile list has at most ceil(N / 128) + batch tiles, so more
  // segments than that would stay empty.
  int64_t nseg = num_cus / pl.HG;
  if (nseg < 1) nseg = 1;
  const int64_t max_tiles = (total_tokens > 0 ? (total_tokens + TILE - 1) / TILE : 0) + batch;
  if (nseg > max_tiles) nseg = max_tiles;
  if (nseg < 1) nseg = 1;
  pl.nseg = (int32_t)nseg;
  pl.items = pl.nseg * pl.HG;
  if (pl.HG > 1) {
    pl.xcd_per = (pl.items + 7) / 8;
    pl.grid = 8 * pl.xcd_per;
  } else {
    pl.xcd_per = pl.items;
    pl.grid = pl.items;
  }
  // Workspace: per-request piece ranges, then partial outputs and
  // log2-sum-exps; pieces are indexed segment + request, fewer than
  // nseg + batch.
  const size_t npieces = (size_t)pl.nseg + (size_t)batch;
  const size_t ranges_bytes = (size_t)batch * 2 * sizeof(int32_t);
  const size_t o_bytes = npieces * pl.Hp * V_WIDTH * sizeof(uint16_t);
  const size_t lse_bytes = npieces * pl.Hp * sizeof(float);
  pl.part_o_offset = (ranges_bytes + 255) / 256 * 256;
  pl.lse_offset = pl.part_o_offset + (o_bytes + 255) / 256 * 256;
  pl.workspace_bytes = pl.lse_offset + (lse_bytes + 255) / 256 * 256;
  return pl;
}

hipError_t launch_mla_decode(const uint16_t* q, const uint8_t* kv_pool, int64_t num_slots,
                             const int32_t* kv_indptr, const int32_t* kv_indices,
                             int64_t total_tokens, int32_t batch, int32_t num_heads, float scale,
                             float sm_scale, uint16_t* out, void* workspace, const DecodePlan& pl,
                             hipStream_t stream) {
  char* ws = reinterpret_cast<char*>(workspace);
  SplitParams sp;
  sp.q = q;
  sp.pool = kv_pool;
  sp.indptr = kv_indptr;
  sp.indices = kv_indices;
  sp.out = out;
  sp.part_o = reinterpret_cast<uint16_t*>(ws + pl.part_o_offset);
  sp.part_lse = reinterpret_cast<float*>(ws + pl.lse_offset);
  sp.req_pieces = total_tokens > 0 ? reinterpret_cast<int2*>(ws) : nullptr;
  sp.max_slot = num_slots > 0 ? (uint32_t)(num_slots - 1) : 0u;
  sp.total_tokens = (int32_t)total_tokens;
  sp.B = batch;
  sp.H = num_heads;
  sp.HG = pl.HG;
  sp.Hp = pl.Hp;
  sp.nseg = pl.nseg;
  sp.items = pl.items;
  sp.xcd_per = pl.xcd_per;
  sp.score_scale = (float)((double)sm_scale * (double)scale * 1.4426950408889634);
  sp.kv_scale = scale;
  hipLaunchKernelGGL(mla_split_kernel, dim3(pl.grid), dim3(THREADS), 0, stream, sp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || total_tokens == 0) return e;  // no tokens: nothing to merge
  CombineParams cp;
  cp.req_pieces = reinterpret_cast<const int2*>(ws);
  cp.part_o = sp.part_o;
  cp.part_lse = sp.part_lse;
  cp.out = out;
  cp.H = num_heads;
  cp.Hp = pl.Hp;
  cp.kv_scale = scale;
  hipLaunchKernelGGL(mla_combine_kernel, dim3(batch, (num_heads + 3) / 4), dim3(256), 0, stream, cp);
  return hipGetLastError();
}

}  // namespace fp8mla
