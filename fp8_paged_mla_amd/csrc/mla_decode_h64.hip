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
//  * wave w owns head group w & 3 and tokens [32(w >> 2), +32) of the tile
//    for the score product S^T = K q^T, two 16-token blocks on the FP8 MFMA
//    16x16x128 (below);
//  * the two waves of a head group exchange maxima and probabilities
//    through LDS;
//  * for P.V, wave w owns output columns [256(w >> 2), +256) of its head
//    group: O^T = V^T P^T over all 64 tokens (16 column blocks of 16, MFMA
//    16x16x32 bf16), with the transposed FP8 value operand read by
//    ds_read_b64_tr_b8.
// Rows are copied global -> LDS (global_load_lds) into three slots of 64
// rows: tile k+2 goes into the slot of tile k-1 once every wave has finished
// tile k-1's value reads (the first barrier of tile k), ~1.5 tiles ahead.
//
// Scores on the FP8 MFMA: v_mfma_f32_16x16x128_f8f6f4 runs at 3.5x the BF16
// MFMA's rate on this part and takes K straight from the FP8 tile: no K
// byte is converted (converting K once per head group was a quarter of the
// kernel's VALU work, which bounds it).  A single E4M3 query would miss the
// attention tolerance, so q_split_kernel first writes per query row the
// codes of q * s (hi) and of the 16x rounding residual (lo), s a power of
// two putting the row's largest magnitude in [224, 448]: hi + lo / 16 keeps
// about 8 significant bits, as BF16 does.  A workgroup keeps its rows' hi
// codes in registers (40 VGPRs per lane) and copies their lo rows into a
// fourth LDS slot like KV rows; scores are (K.hi + K.lo / 16) / s.  Lane
// (t, g) of the MFMA holds bytes 32g .. 32g+31 of each 128-dim chunk for both
// operands (the instruction sums over any common pairing); 576 dims are four
// full chunks and a fifth whose lanes g = 2, 3 repeat dims 512..575 against
// zero hi and lo codes.
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
constexpr int ROWS_PER_WAVE = TILE / NWAVES;      // 8 rows copied by each wave
constexpr int DMA_OPS = (ROWS_PER_WAVE * ROW_SLOTS + 63) / 64;  // 5
constexpr int VBLOCKS = (V_WIDTH / 2) / 16;       // 16 output blocks per wave
static_assert(TILE == 1 << TILE_SHIFT, "tile size");
static_assert(TILE == kH64TileTokens, "host and kernel tile sizes agree");

// Wait until at most n vector-memory operations are outstanding (n is
// wave-uniform and one of the counts this pipeline produces; any other value
// waits for everything).
__device__ __forceinline__ void wait_vm_upto(int n) {
  switch (n) {
    case 1: wait_vm<1>(); break;
    case 5: wait_vm<5>(); break;
    case 6: wait_vm<6>(); break;
    case 11: wait_vm<11>(); break;
    default: wait_vm<0>(); break;
  }
}

constexpr int Q8_CHUNKS = 5;
typedef __attribute__((ext_vector_type(8))) int i32x8_t;
typedef i32x8_t __attribute__((aligned(16))) i32x8_a16_t;  // LDS rows are 16-byte aligned

__device__ __forceinline__ float wave_max64(float x) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

// Codes of 4 values (|x| <= 448), byte j = element j, and of their 16x residuals.
__device__ __forceinline__ void e4m3_hi_lo(float x0, float x1, float x2, float x3, uint32_t& h,
                                           uint32_t& l) {
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
  h = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, r, true);
  const auto b01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)h, false);
  const auto b23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)h, true);
  r = __builtin_amdgcn_cvt_pk_fp8_f32((x0 - b01[0]) * 16.f, (x1 - b01[1]) * 16.f, 0, false);
  l = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32((x2 - b23[0]) * 16.f, (x3 - b23[1]) * 16.f, r, true);
}

// Eight BF16 values (16 bytes) times s -> 8 hi codes and 8 lo codes.
__device__ __forceinline__ void split8(const u32x4_t v, float s, u32x2_t& hi, u32x2_t& lo) {
  uint32_t h0, l0, h1, l1;
  e4m3_hi_lo(bf16_bits_to_f32(v[0] & 0xFFFFu) * s, bf16_bits_to_f32(v[0] >> 16) * s,
             bf16_bits_to_f32(v[1] & 0xFFFFu) * s, bf16_bits_to_f32(v[1] >> 16) * s, h0, l0);
  e4m3_hi_lo(bf16_bits_to_f32(v[2] & 0xFFFFu) * s, bf16_bits_to_f32(v[2] >> 16) * s,
             bf16_bits_to_f32(v[3] & 0xFFFFu) * s, bf16_bits_to_f32(v[3] >> 16) * s, h1, l1);
  hi = u32x2_t{h0, h1};
  lo = u32x2_t{l0, l1};
}

__device__ __forceinline__ float absmax8(const u32x4_t v) {
  float m = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    m = fmaxf(m, fmaxf(fabsf(bf16_bits_to_f32(v[e] & 0xFFFFu)), fabsf(bf16_bits_to_f32(v[e] >> 16))));
  return m;
}

// One wave per query row (576 BF16): lane l takes dims 8l..8l+7, lanes 0..7
// also dims 512+8l..; writes hi and lo codes (576 bytes each) and 1 / s.
constexpr int QSPLIT_ROWS = 4;
__global__ __launch_bounds__(64 * QSPLIT_ROWS) void q_split_kernel(
    const uint16_t* __restrict__ q, int64_t rows, uint8_t* __restrict__ hi,
    uint8_t* __restrict__ lo, float* __restrict__ inv) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * QSPLIT_ROWS + (threadIdx.x >> 6);
  if (row >= rows) return;
  const uint16_t* src = q + row * KV_WIDTH;
  const u32x4_t a = *reinterpret_cast<const u32x4_t*>(src + 8 * lane);
  u32x4_t b = {0u, 0u, 0u, 0u};
  if (lane < 8) b = *reinterpret_cast<const u32x4_t*>(src + 512 + 8 * lane);
  const float amax = wave_max64(fmaxf(absmax8(a), absmax8(b)));
  float s = 1.f;
  if (amax > 0.f && amax <= 3.0e38f)  // 2^(e-1) <= 448 / amax
    s = __builtin_amdgcn_ldexpf(1.f, __builtin_amdgcn_frexp_expf(448.f / amax) - 1);
  u32x2_t h, l;
  split8(a, s, h, l);
  *reinterpret_cast<u32x2_t*>(hi + row * KV_WIDTH + 8 * lane) = h;
  *reinterpret_cast<u32x2_t*>(lo + row * KV_WIDTH + 8 * lane) = l;
  if (lane < 8) {
    split8(b, s, h, l);
    *reinterpret_cast<u32x2_t*>(hi + row * KV_WIDTH + 512 + 8 * lane) = h;
    *reinterpret_cast<u32x2_t*>(lo + row * KV_WIDTH + 512 + 8 * lane) = l;
  }
  if (lane == 0) inv[row] = 1.f / s;
}

// Tile row of MFMA row m of 16-token block B.  Odd blocks use row m ^ 12 so
// that the transposed value reads of two consecutive blocks fall in distinct
// LDS banks.
__device__ __forceinline__ int tile_row(int B, int m) { return 16 * B + ((B & 1) ? (m ^ 12) : m); }

template <bool EXT>
__global__ __launch_bounds__(THREADS) void mla_split_h64_kernel(const SplitParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t kv_lds[NSLOTS * TILE_BYTES];
  // the workgroup's 64 lo query rows (row r at r * ROWB), then 32 zero bytes
  __shared__ __attribute__((aligned(16))) uint8_t qlo_lds[TILE_BYTES + 32];
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
  if (!find_segment<TILE_SHIFT, THREADS, WG_HEADS, !EXT>(p, seg, hs, lane, span)) return;
  const int ntiles = span.ntiles;
  using Cursor = TileCursor<TILE_SHIFT, EXT>;
  Cursor cc;
  cc.start(p, span.b0, span.j0, lane);
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
    int off = 0;  // extend: CSR position -> kv_indices entry
    if constexpr (EXT) off = lc.delta;
    const int32_t* a = lc.nt > 0 ? p.indices + (tok < lc.tile_hi() ? tok : tlo) + off : p.indices;
    const int32_t v = issue_load_i32(a);
    lc.advance(p, lane);
    return v;
  };
  const uint32_t lds_tiles = (uint32_t)(uintptr_t)(
      (__attribute__((address_space(3))) uint8_t*)&kv_lds[0]);
  // rows 8w .. 8w+7 of a 64-row block into LDS at `lds_block`: op j fills
  // 16-byte LDS chunks 64j .. 64j+63 of the wave's block of 8 x 37 (row P /
  // 37, chunk P % 37; the pad chunk gets a copy of chunk 35; lanes past the
  // block masked off).  Row 8w + i comes from src + idx * 576, idx held by
  // lane i (clamped to max_idx).
  auto issue_rows = [&](const uint8_t* src, uint32_t max_idx, uint32_t lds_block, int32_t idx) {
    const uint32_t base = __builtin_amdgcn_readfirstlane(lds_block + (uint32_t)(ROWS_PER_WAVE * w * ROWB));
    const int ln = opaque_lane();
#pragma unroll
    for (int j = 0; j < DMA_OPS; ++j) {
      const int P = 64 * j + ln;
      const int r = P / ROW_SLOTS;
      const int c = min(P - r * ROW_SLOTS, KV_CHUNKS - 1);
      const uint32_t s = (uint32_t)__shfl(idx, r & 7);
      const uint8_t* a = src + (uint64_t)(s < max_idx ? s : max_idx) * KV_WIDTH + 16 * c;
      if (j < DMA_OPS - 1 || P < ROWS_PER_WAVE * ROW_SLOTS) issue_lds_dma16(a, base + 1024 * j);
    }
  };
  auto issue_tile = [&](int slot, int32_t idx) {
    issue_rows(p.pool, p.max_slot, lds_tiles + (uint32_t)(slot * TILE_BYTES), idx);
  };

  // query of this wave's head group, in the d-order of the K reads: step
  // s = 2i + e, lane (t, g): q[head t][64i + 16g + 8e .. +8]
  // query row index (query token * H + head) of workgroup row r (0..63)
  // of request c; rows without a query map to a valid row
  auto row_index = [&](const Cursor& c, int r) -> int64_t {
    int64_t qrow = c.b;
    int h = hs * WG_HEADS + r, k = 0;
    if constexpr (EXT) {
      if (p.rows_per_tok > 0) {
        k = r / p.rows_per_tok;
        h = r - k * p.rows_per_tok;
      }
      qrow = c.q_row0() + min(k, c.q_tokens() - 1);
    }
    return qrow * p.H + min(h, p.H - 1);
  };
  // rows without a query (heads past H; extend: tokens past the block) keep a zero query
  auto row_idle = [&]() -> bool {
    if constexpr (EXT) return head >= p.H || tk >= cc.q_tokens();
    return head >= p.H;
  };
  i32x8_t qh[Q8_CHUNKS];  // hi codes of this lane's query row, per 128-dim chunk
  float q_inv = 1.f;      // 1 / s of this lane's row
  const uint32_t qlo_base = (uint32_t)(uintptr_t)(
      (__attribute__((address_space(3))) uint8_t*)&qlo_lds[0]);
  // issue the lo query rows of request c into LDS (DMA_OPS memory ops)
  auto issue_q = [&](const Cursor& c) {
    const int64_t ri = row_index(c, ROWS_PER_WAVE * w + (t & 7));
    issue_rows(p.q_lo, 0xFFFFFFFFu, qlo_base, (int32_t)ri);
  };
  // this wave's lo rows have landed (the caller synchronises the workgroup
  // before they are read): load the hi codes and 1 / s of this lane's row
  auto finish_q = [&]() {
    const int64_t ri = row_index(cc, hgl * HEADS + t);
    const uint8_t* hp = p.q_hi + ri * KV_WIDTH;
    const bool idle = row_idle();
#pragma unroll
    for (int c = 0; c < Q8_CHUNKS; ++c) {
      const int off = c < Q8_CHUNKS - 1 ? 128 * c + 32 * g : 512 + 32 * (g & 1);
      const i32x8_t v = *reinterpret_cast<const i32x8_t*>(hp + off);
      qh[c] = idle || (c == Q8_CHUNKS - 1 && g >= 2) ? i32x8_t{} : v;
    }
    q_inv = p.q_inv[ri];
  };

  // Prologue: indices of tiles 0 and 1; query, rows of tile 0, index of tile
  // 2, rows of tile 1.  "At most 6 outstanding" proves query and tile 0.
  int32_t ixA = load_next_index();  // tile k % 2 == 0: index of tile k + 2
  int32_t ixB = load_next_index();
  wait_vm<0>();
  pin(ixA);
  pin(ixB);
  // 32 zero bytes after the lo rows (the fifth chunk's lanes g = 2, 3)
  if (threadIdx.x < 8) reinterpret_cast<uint32_t*>(qlo_lds + TILE_BYTES)[threadIdx.x] = 0u;
  issue_q(cc);
  issue_tile(0, ixA);
  ixA = load_next_index();
  if (ntiles > 1) issue_tile(1, ixB);
  wait_vm_upto(ntiles > 1 ? 1 + DMA_OPS : 1);
  finish_q();
  __syncthreads();

  // LDS offsets.  Scores: block B = 2 half + b, lane (t, g) reads chunk 4i + g
  // of tile row tile_row(B, t).  Values: as in the 16-head kernel with the
  // wave's column base 256 half.
  const int k_row0 = tile_row(2 * half, t) * ROWB;
  const int k_row1 = tile_row(2 * half + 1, t) * ROWB;
  const int qlo_row = (hgl * HEADS + t) * ROWB;  // this lane's row of the lo block
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
      p.req_pieces[cc.b] = make_int2(s0, s1 - s0 + 1);
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
      const int64_t piece = (int64_t)(seg + cc.b) * p.Hp + row;
      const bool empty = EXT && l == 0.f;  // extend: no visible token in this piece
      const float inv = empty ? 0.f : 1.0f / l;
      uint16_t* op = p.part_o + piece * V_WIDTH + 256 * half + 4 * g;
#pragma unroll
      for (int c = 0; c < VBLOCKS; ++c)
        *reinterpret_cast<uint2*>(op + 16 * c) =
            make_uint2(pack_f16x2(O[c][0] * inv, O[c][1] * inv), pack_f16x2(O[c][2] * inv, O[c][3] * inv));
      if (half == 0 && g == 0) p.part_lse[piece] = empty ? -INFINITY : m_run + __builtin_amdgcn_logf(l);
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
      __syncthreads();  // every wave's lo rows landed
      q_pending = false;
    }

    // a0 / c0 from the hi codes, a1 / c1 from the lo codes (weight 1/16)
    f32x4_t a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0, c0 = a0, c1 = a0;
    const uint8_t* kp0 = slot + k_row0;
    const uint8_t* kp1 = slot + k_row1;
#pragma unroll
    for (int c = 0; c < Q8_CHUNKS; ++c) {
      const int ko = c < Q8_CHUNKS - 1 ? 128 * c + 32 * g : 512 + 32 * (g & 1);
      const i32x8_t k0 = *reinterpret_cast<const i32x8_a16_t*>(kp0 + ko);
      const i32x8_t k1 = *reinterpret_cast<const i32x8_a16_t*>(kp1 + ko);
      const i32x8_t ql = *reinterpret_cast<const i32x8_a16_t*>(
          qlo_lds + (c < Q8_CHUNKS - 1 || g < 2 ? qlo_row + ko : TILE_BYTES));
      a0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(k0, qh[c], a0, 0, 0, 0, 0, 0, 0);
      a1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(k0, ql, a1, 0, 0, 0, 0, 0, 0);
      c0 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(k1, qh[c], c0, 0, 0, 0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(k1, ql, c1, 0, 0, 0, 0, 0, 0);
    }
    const float sc0 = p.score_scale * q_inv, sc1 = sc0 * 0.0625f;
    float s0[4], s1[4];
    float lmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      s0[r] = tile_lo + s_tok0 + r < tile_hi ? a0[r] * sc0 + a1[r] * sc1 : -INFINITY;
      s1[r] = tile_lo + s_tok1 + r < tile_hi ? c0[r] * sc0 + c1[r] * sc1 : -INFINITY;
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
      issue_q(nc);
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
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pr0[r] = __builtin_amdgcn_exp2f(s0[r] - m_sub);
      pr1[r] = __builtin_amdgcn_exp2f(s1[r] - m_sub);
    }
    const uint32_t p01 = pack_bf16x2(pr0[0], pr0[1]), p23 = pack_bf16x2(pr0[2], pr0[3]);
    const uint32_t q01 = pack_bf16x2(pr1[0], pr1[1]), q23 = pack_bf16x2(pr1[2], pr1[3]);
    l_w += (bf16_bits_to_f32(p01 & 0xFFFFu) + bf16_bits_to_f32(p01 >> 16)) +
           (bf16_bits_to_f32(p23 & 0xFFFFu) + bf16_bits_to_f32(p23 >> 16)) +
           (bf16_bits_to_f32(q01 & 0xFFFFu) + bf16_bits_to_f32(q01 >> 16)) +
           (bf16_bits_to_f32(q23 & 0xFFFFu) + bf16_bits_to_f32(q23 >> 16));
    p_lds[w][0][lane] = make_uint2(p01, p23);
    p_lds[w][1][lane] = make_uint2(q01, q23);
    // rows of tile k+1 landed (younger: index k+3, maybe a query, rows k+2)
    if (k + 1 < ntiles) wait_vm_upto(1 + (new_q ? DMA_OPS : 0) + (k + 2 < ntiles ? DMA_OPS : 0));
    __syncthreads();

    // P.V over the tile's 64 tokens: step st covers blocks 2st and 2st+1,
    // whose probabilities the wave (hgl, st) produced
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const uint2 x = p_lds[hgl + 4 * st][0][lane];
      const uint2 y = p_lds[hgl + 4 * st][1][lane];
      const u32x4_t pv = {x.x, x.y, y.x, y.y};
      const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pv);
      const uint8_t* vb = slot + tr_off + 32 * ROWB * st;
#pragma unroll
      for (int c = 0; c < VBLOCKS; ++c) {
        const i32x2_t vt = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (__attribute__((address_space(3))) i32x2_t*)(vb + 16 * c));
        O[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16x8((uint32_t)vt.x, (uint32_t)vt.y),
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
  decode::SplitParams sp = make_split_params(q, kv_pool, num_slots, kv_indptr, kv_indices,
                                             total_tokens, batch, num_heads, scale, sm_scale, out,
                                             workspace, pl);
  hipError_t e = launch_q_split(q, (int64_t)batch * num_heads,
                                reinterpret_cast<char*>(workspace) + pl.q8_offset, sp, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mla_split_h64_kernel<false>, dim3(pl.grid), dim3(THREADS), 0, stream, sp);
  e = hipGetLastError();
  if (e != hipSuccess || total_tokens == 0) return e;
  return launch_mla_combine(sp, stream);
}

hipError_t launch_mla_split_h64_extend(const decode::SplitParams& sp, int grid, hipStream_t stream) {
  hipLaunchKernelGGL(mla_split_h64_kernel<true>, dim3(grid), dim3(THREADS), 0, stream, sp);
  return hipGetLastError();
}

hipError_t launch_q_split(const uint16_t* q, int64_t rows, void* buffers, decode::SplitParams& sp,
                          hipStream_t stream) {
  const Q8Buffers qb = q8_buffers(buffers, rows);
  sp.q_hi = qb.hi;
  sp.q_lo = qb.lo;
  sp.q_inv = qb.inv;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(q_split_kernel, dim3((unsigned)((rows + QSPLIT_ROWS - 1) / QSPLIT_ROWS)),
                     dim3(64 * QSPLIT_ROWS), 0, stream, q, rows, qb.hi, qb.lo, qb.inv);
  return hipGetLastError();
}

}  // namespace fp8mla
