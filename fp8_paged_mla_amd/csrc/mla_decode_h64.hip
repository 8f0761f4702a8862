// Split-K MLA decode over a paged FP8-E4M3FN latent cache for high head
// counts (64 or more query heads per KV head), for gfx950.
//
// Same computation, work split, partial format and combine as the 16-head
// kernel (mla_decode.hip); what changes is the work inside a workgroup.  With
// 16 heads per workgroup, H = 128 needs eight workgroups per segment, each of
// which copies every tile and pays the per-tile latencies for one 16-head
// slice of the math.  Here one workgroup (8 waves) takes 64 heads (four
// groups of 16) over 64-token tiles, so a tile is copied and exchanged once
// per 64 heads and each wave issues four times the MFMA work per tile:
//  * wave w owns head group w & 3 (its 16 heads' query in registers) and
//    tokens [32(w >> 2), +32) of the tile for the score product
//    S^T = K q^T (MFMA 16x16x32 bf16, two 16-token blocks);
//  * the two waves of a head group exchange maxima and probabilities
//    through LDS;
//  * for P.V, wave w owns output columns [256(w >> 2), +256) of its head
//    group: O^T = V^T P^T over all 64 tokens (16 column blocks of 16, MFMA
//    16x16x32 f16 on FP16 probabilities), with the transposed FP8 value
//    operand read by ds_read_b64_tr_b8.
// Rows are copied global -> LDS (global_load_lds) into three slots of 64
// rows: tile k+2 goes into the slot of tile k-1 once every wave has finished
// tile k-1's value reads (the first barrier of tile k), ~1.5 tiles ahead.
//
// The extend instantiation (EXT) serves several query tokens per request:
// the 64 rows of a workgroup are (token, head) pairs of one virtual request
// (a request and a block of its query tokens, built on the device), so every
// KV tile is shared by the block's tokens as it is by the heads.  A wave's 16
// rows belong to one token, whose causal limit masks the scores; a token
// without visible tokens in a piece yields an empty partial (lse -inf).
#include "decode_host.h"

namespace fp8mla {
namespace {

using namespace decode;

constexpr int NWAVES = 8;
constexpr int THREADS = 64 * NWAVES;              // 512
constexpr int GROUPS = 4;                         // head groups of 16 per workgroup
constexpr int WG_HEADS = GROUPS * HEADS;          // 64
constexpr int TILE = 64;                          // tokens per tile
constexpr int TILE_SHIFT = 6;
constexpr int NSLOTS = 3;
constexpr int ROW_SLOTS = KV_CHUNKS + 1;          // 37 (odd 16-byte stride)
constexpr int ROWB = 16 * ROW_SLOTS;              // 592
constexpr int TILE_BYTES = TILE * ROWB;           // 37888
constexpr int KSTEPS = KV_WIDTH / 64;             // 9
constexpr int QSTEPS = 2 * KSTEPS;                // 18
constexpr int ROWS_PER_WAVE = TILE / NWAVES;      // 8 rows copied by each wave
constexpr int DMA_OPS = (ROWS_PER_WAVE * ROW_SLOTS + 63) / 64;  // 5
constexpr int VBLOCKS = (V_WIDTH / 2) / 16;       // 16 output blocks per wave
static_assert(TILE == 1 << TILE_SHIFT, "tile size");
static_assert(TILE == kH64TileTokens, "host and kernel tile sizes agree");
static_assert(TILE_SHIFT == kExtendTileShift, "extend's tile CSR counts this kernel's tiles");

__device__ __forceinline__ void issue_load_q(bf16x8_t (&q)[QSTEPS], const uint16_t* qp) {
  // 9 pairs of 16-byte pieces 64 elements (128 bytes) apart
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

__device__ __forceinline__ void pin_q(bf16x8_t (&q)[QSTEPS]) {
  asm volatile(""
               : "+v"(q[0]), "+v"(q[1]), "+v"(q[2]), "+v"(q[3]), "+v"(q[4]), "+v"(q[5]),
                 "+v"(q[6]), "+v"(q[7]), "+v"(q[8]));
  asm volatile(""
               : "+v"(q[9]), "+v"(q[10]), "+v"(q[11]), "+v"(q[12]), "+v"(q[13]), "+v"(q[14]),
                 "+v"(q[15]), "+v"(q[16]), "+v"(q[17]));
}

// Wait until at most n vector-memory operations are outstanding (n is
// wave-uniform and one of the counts this pipeline produces; any other value
// waits for everything).
__device__ __forceinline__ void wait_vm_upto(int n) {
  switch (n) {
    case 1: wait_vm<1>(); break;
    case 5: wait_vm<5>(); break;
    case 6: wait_vm<6>(); break;
    case 19: wait_vm<19>(); break;
    case 24: wait_vm<24>(); break;
    default: wait_vm<0>(); break;
  }
}

// Tile row of MFMA row m of 16-token block B.  Odd blocks use row m ^ 12 so
// that the transposed value reads of two consecutive blocks fall in distinct
// LDS banks.
__device__ __forceinline__ int tile_row(int B, int m) { return 16 * B + ((B & 1) ? (m ^ 12) : m); }

template <bool EXT>
__global__ __launch_bounds__(THREADS) void mla_split_h64_kernel(const SplitParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t kv_lds[NSLOTS * TILE_BYTES];
  __shared__ float mx_lds[NWAVES][HEADS];
  __shared__ uint2 p_lds[NWAVES][2][64];
  __shared__ float l_lds[NWAVES][HEADS];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t = lane & 15;
  const int g = lane >> 4;
  const int hgl = w & 3;   // head group of this wave
  const int half = w >> 2;  // token half (scores) and column half (P.V)

  // p.HG counts sets of 64 heads here
  int item = blockIdx.x;
  if (p.HG > 1) item = (int)(blockIdx.x & 7) * p.xcd_per + (int)(blockIdx.x >> 3);
  if (item >= p.items) return;
  const int seg = item / p.HG;
  const int hs = item - seg * p.HG;
  // row: this lane's row of the workgroup's partial results; decode: the
  // head.  Extend: rows are (token tk of the block, head), 16-row groups never
  // straddle tokens (rows per token is a multiple of 16), so tk is per wave.
  const int row = hs * WG_HEADS + hgl * HEADS + t;
  int head = row, tk = 0;
  if constexpr (EXT) {
    if (p.rows_per_tok > 0) {
      tk = (hgl * HEADS) / p.rows_per_tok;
      head = hgl * HEADS - tk * p.rows_per_tok + t;
    }
  }

  SegmentSpan span;
  // (extend: the virtual requests' CSR counts tiles already)
  if (!find_segment<EXT ? 0 : TILE_SHIFT, THREADS, WG_HEADS, !EXT>(p, seg, hs, lane, span)) return;
  const int ntiles = span.ntiles;
  using Cursor = TileCursor<TILE_SHIFT, EXT>;
  Cursor cc;
  cc.start(p, span, lane);
  Cursor lc = cc;

  auto opaque_lane = [&]() -> int {
    int l = lane;
    asm volatile("" : "+v"(l));
    return l;
  };
  // index of the load cursor's tile: lane l (and copies) holds the slot of
  // row 8w + (l & 7); tokens past the request read the tile's first row
  auto load_next_index = [&]() -> int32_t {
    const int tlo = lc.tile_lo();
    const int tok = tlo + ROWS_PER_WAVE * w + (t & 7);
    const int32_t* a = lc.nt > 0 ? p.indices + (tok < lc.tile_hi() ? tok : tlo) : p.indices;
    const int32_t v = issue_load_i32(a);
    lc.advance(p, lane);
    return v;
  };
  const uint32_t lds_tiles = (uint32_t)(uintptr_t)(
      (__attribute__((address_space(3))) uint8_t*)&kv_lds[0]);
  // rows 8w .. 8w+7 of a tile into a slot: op j fills 16-byte LDS chunks
  // 64j .. 64j+63 of the wave's block of 8 x 37 (row P / 37, chunk P % 37;
  // the pad chunk gets a copy of chunk 35; lanes past the block masked off)
  auto issue_tile = [&](int slot, int32_t idx) {
    const uint32_t base = __builtin_amdgcn_readfirstlane(
        lds_tiles + (uint32_t)(slot * TILE_BYTES + ROWS_PER_WAVE * w * ROWB));
    const int ln = opaque_lane();
#pragma unroll
    for (int j = 0; j < DMA_OPS; ++j) {
      const int P = 64 * j + ln;
      const int r = P / ROW_SLOTS;
      const int c = min(P - r * ROW_SLOTS, KV_CHUNKS - 1);
      const uint32_t s = (uint32_t)__shfl(idx, r & 7);
      const uint8_t* a = p.pool + (uint64_t)(s < p.max_slot ? s : p.max_slot) * KV_WIDTH + 16 * c;
      if (j < DMA_OPS - 1 || P < ROWS_PER_WAVE * ROW_SLOTS) {
        // decode reads each row once per head group, close together in time
        // (non-temporal hint); extend re-reads a request's rows for each of
        // its query blocks (default policy)
        if constexpr (!EXT) issue_lds_dma16_nt(a, base + 1024 * j);
        else issue_lds_dma16(a, base + 1024 * j);
      }
    }
  };

  // query of this wave's head group, in the d-order of the K reads: step
  // s = 2i + e, lane (t, g): q[head t][64i + 16g + 8e .. +8]
  auto q_lane_ptr = [&](const Cursor& c) -> const uint16_t* {
    int64_t qrow = c.b;
    if constexpr (EXT) qrow = c.q_row0() + min(tk, c.q_tokens() - 1);
    return p.q + (qrow * p.H + min(head, p.H - 1)) * KV_WIDTH + 16 * g;
  };
  // rows without a query (heads past H; extend: tokens past the block) keep a zero query
  auto row_idle = [&]() -> bool {
    if constexpr (EXT) return head >= p.H || tk >= cc.q_tokens();
    return head >= p.H;
  };
  bf16x8_t qr[QSTEPS];
  auto finish_q = [&]() {
    pin_q(qr);
    if (row_idle()) {
#pragma unroll
      for (int s = 0; s < QSTEPS; ++s) qr[s] = bf16x8_t{};
    }
  };

  // Prologue: indices of tiles 0 and 1; query, rows of tile 0, index of tile
  // 2, rows of tile 1.  "At most 6 outstanding" proves query and tile 0.
  int32_t ixA = load_next_index();  // tile k % 2 == 0: index of tile k + 2
  int32_t ixB = load_next_index();
  wait_vm<0>();
  pin(ixA);
  pin(ixB);
  issue_load_q(qr, q_lane_ptr(cc));
  issue_tile(0, ixA);
  ixA = load_next_index();
  if (ntiles > 1) issue_tile(1, ixB);
  wait_vm_upto(ntiles > 1 ? 1 + DMA_OPS : 1);
  finish_q();
  __syncthreads();

  // LDS offsets.  Scores: block B = 2 half + b, lane (t, g) reads chunk 4i + g
  // of tile row tile_row(B, t).  Values: as in the 16-head kernel with the
  // wave's column base 256 half.
  const int k_off0 = tile_row(2 * half, t) * ROWB + 16 * g;
  const int k_off1 = tile_row(2 * half + 1, t) * ROWB + 16 * g;
  const int tr_row0 = (t >> 1) < 4 ? 4 * g + (t >> 1) : 16 + 4 * (g ^ 3) + (t >> 1) - 4;
  const int tr_off = tr_row0 * ROWB + 8 * (t & 1) + 256 * half;
  const int s_tok0 = 32 * half + 4 * g;             // block 2 half (even)
  const int s_tok1 = 32 * half + 16 + 4 * (g ^ 3);  // block 2 half + 1 (odd, XOR 12)

  f32x4_t O[VBLOCKS];
#pragma unroll
  for (int c = 0; c < VBLOCKS; ++c) O[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;
  float l_w = 0.f;
  bool whole_request = span.j0 == 0;
  int P_cur = span.P0;
  auto record_pieces = [&]() {
    if (hs == 0 && threadIdx.x == 0) {
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
    const float l = l_lds[hgl][t] + l_lds[hgl + 4][t];
    // lane (t, g) holds columns 256 half + 16c + 4g + 0..3 of its head
    if (complete) {
      if (!row_idle()) {
        int64_t orow = cc.b;
        if constexpr (EXT) orow = cc.q_row0() + tk;
        // extend: a token with no visible token gets a zero row
        const float inv = EXT && l == 0.f ? 0.f : p.kv_scale / l;
        uint16_t* op = p.out + (orow * p.H + head) * V_WIDTH + 256 * half + 4 * g;
#pragma unroll
        for (int c = 0; c < VBLOCKS; ++c)
          *reinterpret_cast<uint2*>(op + 16 * c) =
              make_uint2(pack_bf16x2(O[c][0] * inv, O[c][1] * inv), pack_bf16x2(O[c][2] * inv, O[c][3] * inv));
      }
    } else {
      const int64_t piece = (int64_t)piece_slot(seg, cc.b == span.b0) * p.Hp + row;
      const bool empty = EXT && l == 0.f;  // extend: no visible token in this piece
      const float inv = empty ? 0.f : 1.0f / l;
      uint16_t* op = p.part_o + piece * V_WIDTH + 256 * half + 4 * g;
#pragma unroll
      for (int c = 0; c < VBLOCKS; ++c)
        *reinterpret_cast<uint2*>(op + 16 * c) =
            make_uint2(pack_f16x2(O[c][0] * inv, O[c][1] * inv), pack_f16x2(O[c][2] * inv, O[c][3] * inv));
      if (half == 0 && g == 0)
        p.part_lse[piece] = empty ? -INFINITY : m_run + __builtin_amdgcn_logf(l) - kPScaleLog2;
    }
#pragma unroll
    for (int c = 0; c < VBLOCKS; ++c) O[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    l_w = 0.f;
    m_run = -INFINITY;
  };

  // Tile k (slot k % 3): scores -> [barrier: maxima] -> index of k+3, the
  // next request's query if tile k+1 starts one (qr is dead until then),
  // rows of k+2 into slot (k+2) % 3 -> probabilities -> rows of k+1 landed ->
  // [barrier: probabilities, tile k+1] -> P.V.
  bool q_pending = false;
  int slot_k = 0;  // k % 3
  auto process_tile = [&](int k, int32_t& ix_cur, int32_t& ix_next) {
    const int tile_lo = cc.tile_lo();
    int tile_hi = cc.tile_hi();
    if constexpr (EXT) {  // this wave's token sees the first lim tokens of the request
      const int len = cc.hi - cc.lo;
      const int lim = p.causal ? len - (cc.q_tokens() - 1 - tk) : len;
      tile_hi = min(tile_hi, cc.lo + max(lim, 0));
    }
    const bool last_of_request = cc.j + 1 == cc.nt;
    const uint8_t* slot = kv_lds + slot_k * TILE_BYTES;
    const int slot_next2 = slot_k == 0 ? 2 : slot_k - 1;  // (k + 2) % 3
    if (q_pending) {  // issued before the rows of tile k+1: those may stay in flight
      wait_vm_upto(k + 1 < ntiles ? DMA_OPS : 0);
      finish_q();
      q_pending = false;
    }

    f32x4_t a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0, c0 = a0, c1 = a0;
    const uint8_t* kp0 = slot + k_off0;
    const uint8_t* kp1 = slot + k_off1;
#pragma unroll
    for (int i = 0; i < KSTEPS; ++i) {
      const u32x4_t kv0 = *reinterpret_cast<const u32x4_t*>(kp0 + 64 * i);
      const u32x4_t kv1 = *reinterpret_cast<const u32x4_t*>(kp1 + 64 * i);
      a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16x8(kv0[0], kv0[1]), qr[2 * i], a0, 0, 0, 0);
      c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16x8(kv1[0], kv1[1]), qr[2 * i], c0, 0, 0, 0);
      a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16x8(kv0[2], kv0[3]), qr[2 * i + 1], a1, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16x8(kv1[2], kv1[3]), qr[2 * i + 1], c1, 0, 0, 0);
    }
    float s0[4], s1[4];
    float lmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      s0[r] = tile_lo + s_tok0 + r < tile_hi ? (a0[r] + a1[r]) * p.score_scale : -INFINITY;
      s1[r] = tile_lo + s_tok1 + r < tile_hi ? (c0[r] + c1[r]) * p.score_scale : -INFINITY;
      lmax = fmaxf(lmax, fmaxf(s0[r], s1[r]));
    }
    lmax = wave_max_over_groups(lmax);
    if (g == 0) mx_lds[w][t] = lmax;
    __syncthreads();

    wait_vm_upto(k + 1 < ntiles ? DMA_OPS : 0);  // index of tile k+2 arrived
    pin(ix_cur);
    ix_next = load_next_index();
    const bool new_q = last_of_request && k + 1 < ntiles;
    Cursor nc = cc;
    if (new_q) {
      nc.advance(p, lane);
      issue_load_q(qr, q_lane_ptr(nc));
    }
    if (k + 2 < ntiles) issue_tile(slot_next2, ix_cur);

    const float tmax = fmaxf(mx_lds[hgl][t], mx_lds[hgl + 4][t]);
    const float m_new = fmaxf(m_run, tmax);
    // extend: while a token has seen nothing (m -inf), subtract 0 instead
    const float m_sub = EXT && m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_sub);
    if (__ballot(alpha != 1.0f)) {
#pragma unroll
      for (int c = 0; c < VBLOCKS; ++c) O[c] *= alpha;
      l_w *= alpha;
    }
    m_run = m_new;
    float pr0[4], pr1[4];
    const float m_p = m_sub - kPScaleLog2;  // probabilities scaled by 2^15 (FP16 P.V)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pr0[r] = __builtin_amdgcn_exp2f(s0[r] - m_p);
      pr1[r] = __builtin_amdgcn_exp2f(s1[r] - m_p);
    }
    const uint32_t p01 = pack_f16x2(pr0[0], pr0[1]), p23 = pack_f16x2(pr0[2], pr0[3]);
    const uint32_t q01 = pack_f16x2(pr1[0], pr1[1]), q23 = pack_f16x2(pr1[2], pr1[3]);
    l_w += (f16_lo(p01) + f16_hi(p01)) + (f16_lo(p23) + f16_hi(p23)) +
           (f16_lo(q01) + f16_hi(q01)) + (f16_lo(q23) + f16_hi(q23));
    p_lds[w][0][lane] = make_uint2(p01, p23);
    p_lds[w][1][lane] = make_uint2(q01, q23);
    // rows of tile k+1 landed (younger: index k+3, maybe a query, rows k+2)
    if (k + 1 < ntiles) wait_vm_upto(1 + (new_q ? QSTEPS : 0) + (k + 2 < ntiles ? DMA_OPS : 0));
    __syncthreads();

    // P.V over the tile's 64 tokens: step st covers blocks 2st and 2st+1,
    // whose probabilities the wave (hgl, st) produced
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const uint2 x = p_lds[hgl + 4 * st][0][lane];
      const uint2 y = p_lds[hgl + 4 * st][1][lane];
      const u32x4_t pv = {x.x, x.y, y.x, y.y};
      const f16x8_t pb = __builtin_bit_cast(f16x8_t, pv);
      const uint8_t* vb = slot + tr_off + 32 * ROWB * st;
#pragma unroll
      for (int c = 0; c < VBLOCKS; ++c) {
        const i32x2_t vt = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (__attribute__((address_space(3))) i32x2_t*)(vb + 16 * c));
        O[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(e4m3x8_to_f16x8((uint32_t)vt.x, (uint32_t)vt.y),
                                                      pb, O[c], 0, 0, 0);
      }
    }

    if (last_of_request || k + 1 == ntiles) finish_request(whole_request && last_of_request);
    if (new_q) {
      P_cur += TILE_W * cc.nt + START_W;
      cc = nc;
      whole_request = true;
      record_pieces();
      q_pending = true;
    } else {
      cc.advance(p, lane);
    }
    slot_k = slot_k == 2 ? 0 : slot_k + 1;
  };

  for (int k = 0; k < ntiles; k += 2) {
    process_tile(k, ixA, ixB);
    if (k + 1 >= ntiles) break;
    process_tile(k + 1, ixB, ixA);
  }
  wait_vm<0>();  // retire index loads issued past the last tile
}

}  // namespace

hipError_t launch_mla_decode_h64(const uint16_t* q, const uint8_t* kv_pool, int64_t num_slots,
                                 const int32_t* kv_indptr, const int32_t* kv_indices,
                                 int64_t total_tokens, int32_t batch, int32_t num_heads,
                                 float scale, float sm_scale, uint16_t* out, void* workspace,
                                 const DecodePlan& pl, hipStream_t stream) {
  const decode::SplitParams sp = make_split_params(q, kv_pool, num_slots, kv_indptr, kv_indices,
                                                   total_tokens, batch, num_heads, scale,
                                                   sm_scale, out, workspace, pl);
  hipLaunchKernelGGL(mla_split_h64_kernel<false>, dim3(pl.grid), dim3(THREADS), 0, stream, sp);
  hipError_t e = hipGetLastError();
  // no tokens, or one segment (every request complete in it): nothing to merge
  if (e != hipSuccess || total_tokens == 0 || pl.nseg == 1) return e;
  return launch_mla_combine(sp, stream);
}

hipError_t launch_mla_split_h64_extend(const decode::SplitParams& sp, int grid, hipStream_t stream) {
  hipLaunchKernelGGL(mla_split_h64_kernel<true>, dim3(grid), dim3(THREADS), 0, stream, sp);
  return hipGetLastError();
}

}  // namespace fp8mla
