// Pieces shared by the split-K MLA decode kernels (FP8 and BF16 KV rows) of
// libfp8mla.so: the work split over request tiles, the tile cursor, the
// explicitly pipelined memory operations and the merge of partial results.
#pragma once

#include "device_common.h"

#include <math.h>

namespace fp8mla {
namespace decode {

constexpr int HEADS = 16;   // query heads per workgroup (the MFMA N dimension)
constexpr int TILE_W = 4;   // segment balancing: weight of a tile
constexpr int START_W = 2;  // extra weight of a request's first tile

// Extend calls small enough for the split kernel to lay out its list of
// virtual requests itself (extend_common.h): the call's own index arrays and
// where the list goes.  qo_indptr null: the pre-pass kernel built the list.
struct ExtendList {
  const int32_t* qo_indptr;
  const int32_t* kv_indptr;
  int32_t* indptr_out;  // the list's CSR (SplitParams::indptr)
  int2* vinfo_out;      // SplitParams::vinfo
  int32_t* hdr;         // {virtual requests, CSR total}, for the combine
  int32_t batch, total_q, total_kv, T;
};

struct SplitParams {
  const uint16_t* q;
  const uint8_t* pool;      // KV rows (E4M3FN bytes or BF16 bits)
  const int32_t* indptr;
  const int32_t* indices;
  uint16_t* out;
  uint16_t* part_o;         // fp16 bits
  float* part_lse;
  int2* req_pieces;         // per request: (slot of its first piece, number of pieces)
  uint32_t max_slot;
  int32_t total_tokens;
  int32_t B;
  int32_t H;
  int32_t HG;
  int32_t Hp;
  int32_t nseg;     // segments the tile list is cut into (at most)
  int32_t items;    // nseg * HG
  int32_t xcd_per;
  float score_scale;  // sm_scale * scale * log2(e): scores in the base-2 domain
  float kv_scale;
  // Extend (several query tokens per request) only.  The kernels then walk
  // virtual requests, one per (request, block of query tokens), built on the
  // device: indptr is their CSR of tile counts (64-token tiles of the tokens
  // each one sees, padded with empty requests up to B), and per virtual
  // request vinfo holds (its first kv_indices entry, first query row |
  // (tokens in the block - 1) << 23 | (tokens in its last tile - 1) << 25).
  const int2* vinfo;
  int32_t rows_per_tok;  // query rows per token (heads rounded up to 16) if <= 64, else 0
  int32_t causal;
  ExtendList list;
};

// P.V runs in FP16 (the FP16 MFMA is as fast as the BF16 one): the E4M3
// values are exact in FP16, and a probability keeps 11 significant bits
// instead of BF16's 8, so that values of opposite sign up to 448 that cancel
// leave a rounding error well inside the tolerance.  Probabilities are
// formed as exp2(s - m + kPScaleLog2), i.e. scaled by 2^15 into [0, 2^15], so
// that they stay normal FP16 numbers down to 2^-29 of the row maximum; the
// scale cancels in O / l and is taken out of the log-sum-exp of a partial.
constexpr float kPScaleLog2 = 15.0f;

// Fields of vinfo.y (extend): first query row (23 bits), tokens in the block
// - 1 (2 bits), tokens in the last tile - 1 (6 bits).
constexpr int kExtQ0Bits = 23;
constexpr int kExtQ0Mask = (1 << kExtQ0Bits) - 1;
constexpr int kExtTokShift = 23;
constexpr int kExtTailShift = 25;

// Reductions over the four 16-lane rows of a wave (lanes h, h+16, h+32,
// h+48 hold the same head) with the cross-row swaps of gfx950: swap32(a, b)
// gives (a's lanes 0-31 in both halves, b's lanes 32-63 in both halves) when
// a and b hold the same value, swap16 likewise for rows 0/1 and 2/3, so an
// elementwise op of the two results combines lanes l and l^32 (l^16) in every
// lane.  The second operand goes through an opaque copy: given one value
// twice, the compiler folds the two results into one, which is not what the
// instruction does.
struct RowPair {
  float a, b;
};
__device__ __forceinline__ RowPair swap_rows32(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x), v = u;
  asm volatile("" : "+v"(v));
  const auto r = __builtin_amdgcn_permlane32_swap(u, v, false, false);
  return {__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1])};
}
__device__ __forceinline__ RowPair swap_rows16(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x), v = u;
  asm volatile("" : "+v"(v));
  const auto r = __builtin_amdgcn_permlane16_swap(u, v, false, false);
  return {__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1])};
}
// Output rows from P.V accumulators in the MFMA's O^T layout, where lane
// (t, g) holds columns 16c + 4g .. 16c + 4g + 3 of row t for each 16-column
// block c.  Stored as they are, that is 8 bytes per lane and 32 contiguous
// bytes per row and instruction; such stores measured up to 16% slower than
// 16-byte ones on calls with many requests (the 64-row kernel at 64 heads,
// requests of 128 to 4,096 tokens).  Lanes g and g ^ 1 therefore trade a
// block: pair_blocks takes the packed columns of blocks 2k (a) and 2k + 1 (b)
// and returns the 8 consecutive columns that start at 32k + paired_col(g),
// lane g even keeping its block-2k half and taking its partner's, lane g odd
// the same for block 2k + 1.  A store then writes 16 bytes per lane and 64
// contiguous bytes per row.  Every lane of the wave must take part.
__device__ __forceinline__ uint4 pair_blocks(uint2 a, uint2 b) {
  // v_permlane16_swap: the odd 16-lane rows of the first operand trade with
  // the even rows of the second
  const auto x = __builtin_amdgcn_permlane16_swap(a.x, b.x, false, false);
  const auto y = __builtin_amdgcn_permlane16_swap(a.y, b.y, false, false);
  return make_uint4((uint32_t)x[0], (uint32_t)y[0], (uint32_t)x[1], (uint32_t)y[1]);
}
__device__ __forceinline__ int paired_col(int g) { return 4 * g + 12 * (g & 1); }

// max without the canonicalising fmaxf adds to each operand the compiler
// cannot trace to arithmetic (values loaded, exchanged or merged from two
// paths): one instruction instead of up to three.  IEEE maxNum otherwise: a
// NaN operand yields the other operand.
__device__ __forceinline__ float max_f32(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// max(a, b, c) in one instruction, likewise
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

__device__ __forceinline__ float wave_max_over_groups(float x) {
  const RowPair p = swap_rows32(x);
  const RowPair q = swap_rows16(max_f32(p.a, p.b));
  return max_f32(q.a, q.b);
}

__device__ __forceinline__ float wave_sum_over_groups(float x) {
  const RowPair p = swap_rows32(x);
  const RowPair q = swap_rows16(p.a + p.b);
  return q.a + q.b;
}

__device__ __forceinline__ int clamp_tok(int v, int n) { return v < 0 ? 0 : (v > n ? n : v); }

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

// ---- request tiles.  Request b covers tokens [lo_b, hi_b) with
// lo_b = clamp(kv_indptr[b], 0, N) and hi_b = max(lo_b, clamp(kv_indptr[b+1],
// 0, N)), and has ceil((hi_b - lo_b) / 2^SHIFT) tiles.
template <int SHIFT>
__device__ __forceinline__ int tiles_between(int lo, int hi) {
  return (max(lo, hi) - lo + (1 << SHIFT) - 1) >> SHIFT;
}
template <int SHIFT>
__device__ __forceinline__ int request_tiles(const int32_t* indptr, int b, int B, int N) {
  if (b >= B) return 0;
  return tiles_between<SHIFT>(clamp_tok(indptr[b], N), clamp_tok(indptr[b + 1], N));
}

// ---- the work split.  Tiles are weighted by their cost: TILE_W per tile and
// START_W more for the first tile of a request (the query switch and the
// extra output).  Request b's tile j sits at weighted position
// x = P_b + START_W + TILE_W * j, P_b being the total weight of the requests
// before b; segment s takes the tiles with x in [ceil(s W / n), ceil((s+1) W
// / n)), W the total weight, so tile x belongs to segment floor(x n / W).
// Consecutive tile positions are at most TILE_W + START_W apart, so with at
// most W / (TILE_W + START_W) segments every segment holds a tile and the
// pieces of a request are consecutive segments.  (Weights fit in int: with
// tiles of at least 64 tokens W <= 4 (N / 64 + B) + 2 B < 2^31 for
// N < 2^31 and B <= 2^24, the batch limit the host enforces; for extend,
// whose CSR counts tiles (SHIFT 0), W <= 4 N + 6 B with N <= 2^28 tiles and
// B <= 2^25 virtual requests, the bounds its host checks.)
// floor(a / b) for 0 <= a < 2^53 and 0 < b < 2^31 by one double division
// (a 64-bit integer division is a ~100-instruction VALU routine).  a and b
// are exact doubles and the division is correctly rounded, so the quotient q
// moves by at most q 2^-53 < 1 / b: never onto or across an integer that q
// is not already on, which is the whole distance to any other integer.
__device__ __forceinline__ int div_floor_small(int64_t a, int b) {
  return (int)__builtin_floor((double)a / (double)b);
}

struct SegmentSpan {
  int nseg;    // segments in use
  int W;       // total weight
  int ntiles;  // tiles of this segment
  int b0, j0;  // request and tile of its first tile
  int P0;      // weight of the requests before b0
  int win0;    // per lane: clamp(kv_indptr[min(lane, B)]), the first 64-entry window
  __device__ __forceinline__ int segment_of(int x) const {
    return div_floor_small((int64_t)x * nseg, W);  // x < 2^31, nseg <= CUs: below 2^53
  }
};

// One workgroup's segment, found with two wave-wide scans over the requests
// (64 per step); every wave computes the same result.  Segment 0 also writes
// the zero outputs (and piece records) of requests without tokens, for its
// WG_HEADS heads (head set hg).  Returns false if the segment holds no tile.
template <int SHIFT, int THREADS, int WG_HEADS = HEADS, bool ZERO_EMPTY = true>
__device__ __forceinline__ bool find_segment(const SplitParams& p, int seg, int hg, int lane,
                                             SegmentSpan& sp) {
  const int N = p.total_tokens;
  // The first 64 requests' kv_indptr entries are loaded once, in one memory
  // latency, and serve both passes and the tile cursor's first window: with
  // at most 63 requests no other load precedes the first index load.
  // A decode call with one request needs no load at all: the index contract
  // (indptr[0] = 0, indptr[batch] = total_tokens) fixes kv_indptr = [0, N],
  // and skipping it takes one memory latency off the start of small calls.
  int v0, v1;
  if (p.B == 1 && p.vinfo == nullptr) {
    v0 = lane == 0 ? 0 : N;
    v1 = N;
  } else {
    v0 = clamp_tok(p.indptr[min(lane, p.B)], N);
    v1 = clamp_tok(p.indptr[min(lane + 1, p.B)], N);
  }
  const int nt0 = lane < p.B ? tiles_between<SHIFT>(v0, v1) : 0;
  sp.win0 = v0;
  int W = 0;
  for (int c = 0; c < p.B; c += 64) {
    const int nt = c == 0 ? nt0 : request_tiles<SHIFT>(p.indptr, c + lane, p.B, N);
    W += wave_sum_i32(nt > 0 ? TILE_W * nt + START_W : 0);
    uint64_t empty = seg == 0 ? __ballot(c + lane < p.B && nt == 0) : 0ull;
    while (empty) {
      const int b = c + __builtin_ctzll(empty);
      empty &= empty - 1;
      if (hg == 0 && threadIdx.x == 0 && p.req_pieces) p.req_pieces[b] = make_int2(0, 0);
      if (!ZERO_EMPTY) continue;  // the caller's combine writes those rows
      for (int i = threadIdx.x; i < WG_HEADS * 64; i += THREADS) {
        const int h = hg * WG_HEADS + (i >> 6);
        if (h < p.H)
          *reinterpret_cast<uint4*>(p.out + ((int64_t)b * p.H + h) * V_WIDTH + 8 * (i & 63)) =
              make_uint4(0u, 0u, 0u, 0u);
      }
    }
  }
  const int nseg = min(p.nseg, W / (TILE_W + START_W));
  if (seg >= nseg) return false;
  const int x_lo = div_floor_small((int64_t)seg * W + nseg - 1, nseg);  // ceil(seg W / nseg)
  const int x_hi = div_floor_small((int64_t)(seg + 1) * W + nseg - 1, nseg);
  // global index t0 of the first tile at or after x_lo (its request b0, tile
  // j0, weight P0 before b0) and t1 of the first at or after x_hi
  int t0 = -1, t1 = -1, b0 = 0, j0 = 0, P0 = 0;
  int wcarry = 0, tcarry = 0;
  for (int c = 0; c < p.B && t1 < 0; c += 64) {
    const int nt = c == 0 ? nt0 : request_tiles<SHIFT>(p.indptr, c + lane, p.B, N);
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
  sp.nseg = nseg;
  sp.W = W;
  sp.ntiles = t0 < 0 ? 0 : t1 - t0;
  sp.b0 = b0;
  sp.j0 = j0;
  sp.P0 = P0;
  return sp.ntiles > 0;
}

// Walks the tiles of consecutive requests: request b, tile j of its nt
// tiles, kv_indices range [lo, hi).  Requests without tokens are skipped.
// The kv_indptr values come from a 64-entry window held one entry per lane.
// With EXT the requests are virtual (see SplitParams): the window holds
// their tile CSR, and the cursor takes lo, hi and the query rows from a
// window of vinfo held the same way.
template <bool EXT>
struct CursorExtFields {};  // decode: no extra fields (the cursor must stay in registers)
template <>
struct CursorExtFields<true> {
  int q0n;                   // vinfo.y of the current virtual request
  int win_kv0, win_q0n;      // vinfo window, one entry per lane
  __device__ __forceinline__ int q_row0() const { return q0n & kExtQ0Mask; }
  __device__ __forceinline__ int q_tokens() const { return ((q0n >> kExtTokShift) & 3) + 1; }
  __device__ __forceinline__ int tail() const { return ((q0n >> kExtTailShift) & 63) + 1; }
};

template <int SHIFT, bool EXT = false>
struct TileCursor : CursorExtFields<EXT> {
  int b, j, nt, lo, hi;
  int win, win_val;
  __device__ __forceinline__ int tile_lo() const { return lo + (j << SHIFT); }
  __device__ __forceinline__ int tile_hi() const { return min(tile_lo() + (1 << SHIFT), hi); }

  __device__ __forceinline__ void load_window(const SplitParams& p, int first, int lane) {
    win = first;
    win_val = clamp_tok(p.indptr[min(first + lane, p.B)], p.total_tokens);
    if constexpr (EXT) {
      const int2 vi = p.vinfo[min(first + lane, p.B - 1)];
      this->win_kv0 = vi.x;
      this->win_q0n = vi.y;
    }
  }
  // (every field assigned exactly once on every path, so that the cursor
  // stays in registers)
  __device__ __forceinline__ void set_request(const SplitParams& p, int nb, int lane) {
    const bool valid = nb < p.B;  // past the last request: an empty cursor
    if (valid && nb + 1 - win > 63) load_window(p, nb, lane);
    const int l = __builtin_amdgcn_readlane(win_val, valid ? nb - win : 0);
    const int h = max(l, __builtin_amdgcn_readlane(win_val, valid ? nb + 1 - win : 0));
    b = nb;
    if constexpr (EXT) {
      this->q0n = valid ? __builtin_amdgcn_readlane(this->win_q0n, nb - win) : 0;
      nt = valid ? h - l : 0;
      lo = valid ? __builtin_amdgcn_readlane(this->win_kv0, nb - win) : 0;
      hi = nt > 0 ? lo + ((nt - 1) << SHIFT) + this->tail() : lo;
    } else {
      lo = valid ? l : 0;
      hi = valid ? h : 0;
      nt = valid ? (h - l + (1 << SHIFT) - 1) >> SHIFT : 0;
    }
  }
  __device__ __forceinline__ void start(const SplitParams& p, int b0, int j0, int lane) {
    load_window(p, b0, lane);
    set_request(p, b0, lane);
    j = j0;
  }
  // Same, taking the window at request 0 from the segment search when it
  // covers b0 (decode only: the extend window also carries vinfo).
  __device__ __forceinline__ void start(const SplitParams& p, const SegmentSpan& sp, int lane) {
    if (!EXT && sp.b0 < 63) {
      win = 0;
      win_val = sp.win0;
      set_request(p, sp.b0, lane);
      j = sp.j0;
    } else {
      start(p, sp.b0, sp.j0, lane);
    }
  }
  __device__ __forceinline__ void advance(const SplitParams& p, int lane) {
    if (++j < nt) return;
    j = 0;
    do {
      set_request(p, b + 1, lane);
    } while (nt == 0 && b < p.B);
  }
};

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
// otherwise used by these kernels; an LDS DMA reading M0 right after an SALU
// write of it needs one wait state (the s_nop), which the compiler cannot
// insert into inline assembly itself.
__device__ __forceinline__ void issue_lds_dma16(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(lds_base)
               : "memory", "m0");
}

// The same for bytes read once (non-temporal hint: their lines are not kept
// for reuse).  Measured on MI355X: the gather-cast's rows 7% and the 16-head
// decode's rows (one head group per segment) 1% faster than with the default
// policy; the full-pool cast's input 1% slower.
__device__ __forceinline__ void issue_lds_dma16_nt(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
               :
               : "v"(g), "s"(lds_base)
               : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N));
}

__device__ __forceinline__ void pin(int32_t& x) { asm volatile("" : "+v"(x)); }

// ---- partial results.  A segment writes at most two partial pieces: one for
// its first request (begun in an earlier segment, or continuing past this
// one when it is the segment's only request) and one for its last request
// (continuing past the segment); every other request of the segment lies
// inside it and gets its final output directly.  The partial area therefore
// holds 2 * nseg pieces of Hp rows whatever the batch: slot 2s for the first
// request of segment s, slot 2s + 1 for its last.  A request whose tiles
// span segments s0 .. s0 + np - 1 has its pieces in slot `first` = 2 s0 +
// (0 if it is the first request of s0, else 1), then in slot 2s of every
// later segment s, where it is necessarily the first request.
__device__ __forceinline__ int piece_slot(int seg, bool first_of_segment) {
  return 2 * seg + (first_of_segment ? 0 : 1);
}
__device__ __forceinline__ int nth_piece(int first, int i) {
  return i == 0 ? first : (first & ~1) + 2 * i;
}

// Partial outputs are stored as fp16 (round to
// nearest even) before the per-tensor scale; the rows this library is fed
// hold E4M3 values (|v| <= 448), so the partials, convex combinations of
// them, cannot overflow, and fp16's 11-bit significand is finer than the
// bf16 the merged output is rounded to.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  const f16x2_t v = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float f16_lo(uint32_t w) { return (float)__builtin_bit_cast(f16x2_t, w).x; }
__device__ __forceinline__ float f16_hi(uint32_t w) { return (float)__builtin_bit_cast(f16x2_t, w).y; }

// Merge of the np partial results of a request for one head, by one wave
// (pieces nth_piece(first, i), i < np): out = scale * sum_s w_s o_s / sum_s
// w_s with w_s = 2^(lse_s - max lse).  Pieces are taken eight at a time with
// all their loads issued together (one memory latency per eight pieces) and
// folded in with a running maximum.  Lane l produces output columns
// 8l .. 8l+7.
__device__ __forceinline__ void merge_pieces(const uint16_t* part_o, const float* part_lse, int Hp,
                                             int first, int np, int head, float kv_scale,
                                             uint16_t* op, int lane) {
  const float* lse = part_lse + head;  // piece s at lse[s * Hp]
  const uint16_t* po = part_o + (int64_t)head * V_WIDTH + 8 * lane;
  const int64_t pstride = (int64_t)Hp * V_WIDTH;  // elements between consecutive piece slots
  float M = -INFINITY, den = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int base = 0; base < np; base += 8) {
    const int cnt = min(8, np - base);
    const float lv = lane < cnt ? lse[(int64_t)nth_piece(first, base + lane) * Hp] : -INFINITY;
    uint4 x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)  // u >= cnt re-reads the last piece (in bounds, unused)
      x[u] = *reinterpret_cast<const uint4*>(po + (int64_t)nth_piece(first, base + min(u, cnt - 1)) * pstride);
    float cm = lv;
#pragma unroll
    for (int off = 1; off < 8; off <<= 1) cm = fmaxf(cm, __shfl_xor(cm, off));
    const float m_new = fmaxf(M, __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                                     __builtin_bit_cast(int, cm))));
    // pieces without tokens (lse -inf) weigh nothing; while every piece so
    // far is empty, subtract 0 instead of -inf
    const float m_sub = m_new == -INFINITY ? 0.f : m_new;
    const float r = __builtin_amdgcn_exp2f(M - m_sub);  // 0 on the first chunk
    den *= r;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= r;
    M = m_new;
    const float wl = lane < cnt ? __builtin_amdgcn_exp2f(lv - m_sub) : 0.f;
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
  const float inv = den > 0.f ? kv_scale / den : 0.f;  // no token at all: a zero row
  uint4 v;
  v.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  v.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
  v.z = pack_bf16x2(acc[4] * inv, acc[5] * inv);
  v.w = pack_bf16x2(acc[6] * inv, acc[7] * inv);
  *reinterpret_cast<uint4*>(op + 8 * lane) = v;
}

}  // namespace decode
}  // namespace fp8mla
