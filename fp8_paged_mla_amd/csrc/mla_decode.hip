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
//  * the softmax is exchanged through LDS (wave maxima, then FP16
//    probabilities) so that all waves share one running maximum per head;
//  * wave w owns output columns [64w, 64w+64) of O^T = V^T P^T (MFMA
//    16x16x32 f16, M = 16 columns, N = 16 heads, K = 32 tokens), reading the
//    transposed FP8 value operand with ds_read_b64_tr_b8 and converting it
//    to FP16 (exact): no cross-wave reduction of O.
// KV bytes move from HBM once per head group; each value byte is converted
// once per wave that consumes it.
#include "decode_host.h"

namespace fp8mla {
namespace {

using namespace decode;

constexpr int NWAVES = 8;
constexpr int THREADS = 64 * NWAVES;              // 512
constexpr int TILE = 16 * NWAVES;                 // tokens per tile: 16 per wave
constexpr int TILE_SHIFT = 7;                     // log2(TILE)
constexpr int ROW_SLOTS = KV_CHUNKS + 1;          // 16-byte LDS slots per row: 36 + 1 pad (odd)
constexpr int ROWB = 16 * ROW_SLOTS;              // 592 LDS bytes per row
constexpr int TILE_BYTES = TILE * ROWB;           // 75776
constexpr int KSTEPS = KV_WIDTH / 64;             // 16-byte K reads per lane per tile; query steps / 2
constexpr int QSTEPS = 2 * KSTEPS;                // 18 MFMA steps of 32 dims over 576
constexpr int DMA_OPS = (16 * ROW_SLOTS + 63) / 64;  // LDS-copy ops per wave per tile: 10
static_assert(TILE == 1 << TILE_SHIFT, "tile size");


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

// Token row (tile-relative) held by MFMA row m of wave w.  Odd waves use
// row m ^ 12 so that the transposed LDS reads of two consecutive waves'
// rows fall in distinct banks.
__device__ __forceinline__ int tile_row(int w, int m) { return 16 * w + ((w & 1) ? (m ^ 12) : m); }

// NT_ROWS: copy rows with the non-temporal hint (one head group per
// segment: nothing re-reads them); with several head groups the segment's
// workgroups share its rows through L2 and keep the default policy.
template <bool NT_ROWS>
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
  const int head = hg * HEADS + t;  // head whose scores / outputs this lane carries

  // ---- this segment's tiles (cost-weighted split of the list of all
  // requests' tiles), and a cursor over them
  SegmentSpan span;
  if (!find_segment<TILE_SHIFT, THREADS>(p, seg, hg, lane, span)) return;
  const int ntiles = span.ntiles;
  TileCursor<TILE_SHIFT> cc;  // tile being computed
  cc.start(p, span, lane);
  TileCursor<TILE_SHIFT> lc = cc;  // next tile whose index is loaded

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
  // last tile the load reads entry 0 and is never used, and the cursor stays
  // on the last tile rather than walk the rest of the request list)
  int lc_tile = 0;
  auto load_next_index = [&]() -> int32_t {
    const int tlo = lc.tile_lo();
    const int tok = tlo + 16 * w + t;
    const int32_t* a =
        lc_tile < ntiles && lc.nt > 0 ? p.indices + (tok < lc.tile_hi() ? tok : tlo) : p.indices;
    const int32_t v = issue_load_i32(a);
    if (++lc_tile < ntiles) lc.advance(p, lane);
    return v;
  };
  const uint32_t lds_tiles = (uint32_t)(uintptr_t)(
      (__attribute__((address_space(3))) uint8_t*)&kv_lds[0]);
  // What a lane copies depends on the tile only through the slot ids, so the
  // rest is computed once: per op, the permute address of the lane holding
  // its row's id and the address of its chunk in row 0 of the pool (held
  // opaque, so that they stay in registers).
  uint32_t src_lane[DMA_OPS];
  uint64_t cbase[DMA_OPS];
#pragma unroll
  for (int j = 0; j < DMA_OPS; ++j) {
    const int P = 64 * j + lane;
    const int r = P / ROW_SLOTS;
    const int c = min(P - r * ROW_SLOTS, KV_CHUNKS - 1);
    src_lane[j] = 4u * (uint32_t)(r & 15);
    cbase[j] = (uint64_t)(uintptr_t)(p.pool + 16 * c);
    asm volatile("" : "+v"(src_lane[j]), "+v"(cbase[j]));
  }
  auto issue_tile = [&](int k, int32_t idx) {
    const uint32_t base =
        __builtin_amdgcn_readfirstlane(lds_tiles + (uint32_t)((k & 1) * TILE_BYTES + 16 * w * ROWB));
    uint32_t sid[DMA_OPS];
#pragma unroll
    for (int j = 0; j < DMA_OPS; ++j)
      sid[j] = (uint32_t)__builtin_amdgcn_ds_bpermute((int)src_lane[j], idx);
    const int ln = opaque_lane();
#pragma unroll
    for (int j = 0; j < DMA_OPS; ++j) {
      const uint32_t s = sid[j];  // negative ids compare as large
      const uint8_t* a = reinterpret_cast<const uint8_t*>(
          (uintptr_t)(cbase[j] + (uint64_t)(s < p.max_slot ? s : p.max_slot) * KV_WIDTH));
      if (j < DMA_OPS - 1 || ln < 16 * ROW_SLOTS - 64 * (DMA_OPS - 1)) {
        if constexpr (NT_ROWS) issue_lds_dma16_nt(a, base + 1024 * j);
        else issue_lds_dma16(a, base + 1024 * j);
      }
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
  bool whole_request = span.j0 == 0;  // the current request's first tile is in this segment
  int P_cur = span.P0;                 // weight of the requests before the current one
  // Pieces of a request: the segments its tiles [first, first + nt) fall in.
  // Recorded for the combine by the workgroup holding the request's first
  // tile (head group 0).
  auto record_pieces = [&]() {
    if (hg == 0 && threadIdx.x == 0) {
      const int s0 = span.segment_of(P_cur + START_W);
      const int s1 = span.segment_of(P_cur + START_W + TILE_W * (cc.nt - 1));
      p.req_pieces[cc.b] = make_int2(piece_slot(s0, cc.b == span.b0), s1 - s0 + 1);
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
    // lane (t, g) holds columns 64w + 16c + 4g + 0..3 of head t; lanes g and
    // g ^ 1 pair them up for 16-byte stores (pair_blocks)
    const int col = 64 * w + paired_col(g);  // + 32 k for block pair k
    if (complete) {
      const float inv = p.kv_scale / l;
      uint4 d[2];
#pragma unroll
      for (int k = 0; k < 2; ++k)
        d[k] = pair_blocks(make_uint2(pack_bf16x2(O[2 * k][0] * inv, O[2 * k][1] * inv),
                                      pack_bf16x2(O[2 * k][2] * inv, O[2 * k][3] * inv)),
                           make_uint2(pack_bf16x2(O[2 * k + 1][0] * inv, O[2 * k + 1][1] * inv),
                                      pack_bf16x2(O[2 * k + 1][2] * inv, O[2 * k + 1][3] * inv)));
      if (head < p.H) {
        uint16_t* op = p.out + ((int64_t)cc.b * p.H + head) * V_WIDTH + col;
        *reinterpret_cast<uint4*>(op) = d[0];
        *reinterpret_cast<uint4*>(op + 32) = d[1];
      }
    } else {
      const int64_t piece = (int64_t)piece_slot(seg, cc.b == span.b0) * p.Hp + head;
      const float inv = 1.0f / l;
      uint16_t* op = p.part_o + piece * V_WIDTH + col;
#pragma unroll
      for (int k = 0; k < 2; ++k)
        *reinterpret_cast<uint4*>(op + 32 * k) =
            pair_blocks(make_uint2(pack_f16x2(O[2 * k][0] * inv, O[2 * k][1] * inv),
                                   pack_f16x2(O[2 * k][2] * inv, O[2 * k][3] * inv)),
                        make_uint2(pack_f16x2(O[2 * k + 1][0] * inv, O[2 * k + 1][1] * inv),
                                   pack_f16x2(O[2 * k + 1][2] * inv, O[2 * k + 1][3] * inv)));
      if (w == 0 && g == 0) p.part_lse[piece] = m_run + __builtin_amdgcn_logf(l) - kPScaleLog2;
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
#pragma unroll
    for (int r = 0; r < 4; ++r) s[r] = (a0[r] + a1[r]) * p.score_scale;
    if (tile_lo + TILE > tile_hi) {  // (wave-uniform) a partial tile: mask tokens past its end
#pragma unroll
      for (int r = 0; r < 4; ++r) s[r] = tile_lo + s_tok0 + r < tile_hi ? s[r] : -INFINITY;
    }
    float lmax = wave_max_over_groups(max3f(max3f(s[0], s[1], s[2]), s[3], -INFINITY));
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
    TileCursor<TILE_SHIFT> nc = cc;
    if (new_q) {
      nc.advance(p, lane);
      issue_query_copy(nc.b, lds_tiles + (uint32_t)((k & 1) * TILE_BYTES));
    }
    if (rows_now) issue_tile(k + 2, ix_cur);

    static_assert(NWAVES == 8, "maximum over the waves' maxima");
    const float tmax = max3f(max3f(mx_lds[0][t], mx_lds[1][t], mx_lds[2][t]),
                             max3f(mx_lds[3][t], mx_lds[4][t], mx_lds[5][t]),
                             max_f32(mx_lds[6][t], mx_lds[7][t]));
    const float m_new = max_f32(m_run, tmax);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    if (__ballot(alpha != 1.0f)) {
#pragma unroll
      for (int c = 0; c < 4; ++c) O[c] *= alpha;
      l_w *= alpha;
    }
    m_run = m_new;
    float pr[4];
    const float m_p = m_new - kPScaleLog2;  // probabilities scaled by 2^15 (FP16 P.V)
#pragma unroll
    for (int r = 0; r < 4; ++r) pr[r] = __builtin_amdgcn_exp2f(s[r] - m_p);
    const uint32_t p01 = pack_f16x2(pr[0], pr[1]);
    const uint32_t p23 = pack_f16x2(pr[2], pr[3]);
    // the row sums take the probabilities as rounded for P.V
    const f16x2_t one2 = {(_Float16)1.0f, (_Float16)1.0f};
    l_w = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, p01), one2, l_w, false);
    l_w = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, p23), one2, l_w, false);
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

    f16x8_t pb[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const uint2 x = p_lds[2 * st][lane];
      const uint2 y = p_lds[2 * st + 1][lane];
      u32x4_t v = {x.x, x.y, y.x, y.y};
      pb[st] = __builtin_bit_cast(f16x8_t, v);
    }
    // Rows past the request's end in a partial tile are copies of the tile's
    // first row with probability 0, so their value bytes need no masking.
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        O[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
            e4m3x8_to_f16x8((uint32_t)vt[st][c].x, (uint32_t)vt[st][c].y), pb[st], O[c], 0, 0, 0);

    if (last_of_request || k + 1 == ntiles) finish_request(whole_request && last_of_request);
    if (new_q) {
      P_cur += TILE_W * cc.nt + START_W;
      cc = nc;
      whole_request = true;
      record_pieces();
    } else if (k + 1 < ntiles) {  // (past the last tile the cursor is not needed)
      cc.advance(p, lane);
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
  merge_pieces(p.part_o, p.part_lse, p.Hp, rp.x, rp.y, head, p.kv_scale,
               p.out + ((int64_t)b * p.H + head) * V_WIDTH, threadIdx.x & 63);
}

}  // namespace

DecodePlan plan_mla_decode(int32_t batch, int32_t num_heads, int64_t total_tokens, int num_cus,
                           DecodeKernel kernel, int32_t max_segments) {
  const int tile_tokens = kernel == DecodeKernel::kBf16 ? kBf16TileTokens
                          : kernel == DecodeKernel::kFp8H64 ? kH64TileTokens
                                                            : kFp8TileTokens;
  const int wg_heads = kernel == DecodeKernel::kFp8H64 ? 64 : HEADS;
  DecodePlan pl{};
  pl.kernel = kernel;
  pl.HG = (num_heads + wg_heads - 1) / wg_heads;
  pl.Hp = pl.HG * wg_heads;
  // One workgroup per compute unit in flight; head groups of a segment are
  // separate workgroups that share the segment's rows through L2.  The tile
  // list has at most ceil(N / tile) + batch tiles, so more segments than
  // that would stay empty.
  int64_t nseg = num_cus / pl.HG;
  if (nseg < 1) nseg = 1;
  const int64_t max_tiles =
      (total_tokens > 0 ? (total_tokens + tile_tokens - 1) / tile_tokens : 0) + batch;
  if (nseg > max_tiles) nseg = max_tiles;
  if (batch == 1 && total_tokens > 0) {
    // one request: its tile count is known, and so is the split's own cap on
    // segments (every segment holds at least TILE_W + START_W of the total
    // weight 4 t + 2); a single segment needs no merge, so the combine kernel
    // is not launched
    const int64_t t = (total_tokens + tile_tokens - 1) / tile_tokens;
    const int64_t cap = (decode::TILE_W * t + decode::START_W) / (decode::TILE_W + decode::START_W);
    if (nseg > cap) nseg = cap;
  }
  if (max_segments > 0 && nseg > max_segments) nseg = max_segments;
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
  // log2-sum-exps, two piece slots of Hp rows per segment.  Sized for the
  // most piece rows any call with this batch and head count can use (all CUs
  // in use, and either FP8 kernel where the head count admits both), so that
  // the size does not grow with the number of tokens.
  auto piece_rows_of = [&](DecodeKernel k) -> size_t {
    const int wh = k == DecodeKernel::kFp8H64 ? 64 : HEADS;
    const int64_t hg = (num_heads + wh - 1) / wh;
    const int64_t segs = num_cus / hg > 1 ? num_cus / hg : 1;
    return 2 * (size_t)segs * (size_t)(hg * wh);
  };
  size_t piece_rows = piece_rows_of(kernel);
  if (kernel != DecodeKernel::kBf16 && num_heads >= kH64MinHeads) {
    const size_t a = piece_rows_of(DecodeKernel::kFp8), b = piece_rows_of(DecodeKernel::kFp8H64);
    piece_rows = a > b ? a : b;
  }
  const size_t ranges_bytes = (size_t)batch * 2 * sizeof(int32_t);
  const size_t o_bytes = piece_rows * V_WIDTH * sizeof(uint16_t);
  const size_t lse_bytes = piece_rows * sizeof(float);
  pl.part_o_offset = (ranges_bytes + 255) / 256 * 256;
  pl.lse_offset = pl.part_o_offset + (o_bytes + 255) / 256 * 256;
  pl.workspace_bytes = pl.lse_offset + (lse_bytes + 255) / 256 * 256;
  return pl;
}

decode::SplitParams make_split_params(const uint16_t* q, const void* kv_rows, int64_t num_slots,
                                      const int32_t* kv_indptr, const int32_t* kv_indices,
                                      int64_t total_tokens, int32_t batch, int32_t num_heads,
                                      float scale, float sm_scale, uint16_t* out,
                                      void* workspace, const DecodePlan& pl) {
  char* ws = reinterpret_cast<char*>(workspace);
  decode::SplitParams sp{};
  sp.q = q;
  sp.pool = reinterpret_cast<const uint8_t*>(kv_rows);
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
  return sp;
}

hipError_t launch_mla_combine(const decode::SplitParams& sp, hipStream_t stream) {
  CombineParams cp;
  cp.req_pieces = sp.req_pieces;
  cp.part_o = sp.part_o;
  cp.part_lse = sp.part_lse;
  cp.out = sp.out;
  cp.H = sp.H;
  cp.Hp = sp.Hp;
  cp.kv_scale = sp.kv_scale;
  hipLaunchKernelGGL(mla_combine_kernel, dim3(sp.B, (sp.H + 3) / 4), dim3(256), 0, stream, cp);
  return hipGetLastError();
}

hipError_t launch_mla_decode(const uint16_t* q, const uint8_t* kv_pool, int64_t num_slots,
                             const int32_t* kv_indptr, const int32_t* kv_indices,
                             int64_t total_tokens, int32_t batch, int32_t num_heads, float scale,
                             float sm_scale, uint16_t* out, void* workspace, const DecodePlan& pl,
                             hipStream_t stream) {
  if (pl.kernel == DecodeKernel::kFp8H64)
    return launch_mla_decode_h64(q, kv_pool, num_slots, kv_indptr, kv_indices, total_tokens, batch,
                                 num_heads, scale, sm_scale, out, workspace, pl, stream);
  const decode::SplitParams sp = make_split_params(q, kv_pool, num_slots, kv_indptr, kv_indices,
                                                   total_tokens, batch, num_heads, scale,
                                                   sm_scale, out, workspace, pl);
  if (pl.HG == 1)
    hipLaunchKernelGGL(mla_split_kernel<true>, dim3(pl.grid), dim3(THREADS), 0, stream, sp);
  else
    hipLaunchKernelGGL(mla_split_kernel<false>, dim3(pl.grid), dim3(THREADS), 0, stream, sp);
  hipError_t e = hipGetLastError();
  // no tokens, or one segment (every request complete in it): nothing to merge
  if (e != hipSuccess || total_tokens == 0 || pl.nseg == 1) return e;
  return launch_mla_combine(sp, stream);
}

}  // namespace fp8mla
