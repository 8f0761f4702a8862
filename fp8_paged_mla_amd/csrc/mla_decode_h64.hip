// Split-K MLA decode and extend over a paged FP8-E4M3FN latent cache for
// high head counts (64 query heads per workgroup), for gfx950, with the
// workgroup's waves specialised by role.
//
// Same computation, work split, partial format and combine as the 16-head
// kernel (mla_decode.hip).  With 64 heads per KV row the work per row is
// dense (2 x 64 x 1088 flops per token against 576 bytes), so the kernel is
// bound by its matrix and conversion work rather than by HBM.  Two choices
// follow from that:
//  * Roles.  Waves 0-3 ("score waves") each own one head group of 16 heads
//    over the whole tile: S^T = K q^T (MFMA 16x16x32 bf16, K converted from
//    FP8 in registers, the group's query held in registers), their own online
//    softmax (every token of the tile belongs to the wave, so no maximum is
//    exchanged), and FP16 probabilities written to LDS.  Waves 4-11 ("value
//    waves") each own 64 output columns of all 64 heads: O^T = V^T P^T
//    (MFMA 16x16x32 f16), each value byte read transposed
//    (ds_read_b64_tr_b8) and converted once for the four head groups.  A
//    score wave never holds output accumulators and a value wave never holds
//    a query, which keeps both within 168 registers at three waves per SIMD,
//    one score and two value waves, so that one's matrix work and another's
//    conversions can run while the third waits.
//  * Half-tile pipeline.  Time is cut into half-tile intervals (32 tokens)
//    separated by one workgroup barrier: in interval h the score waves
//    produce the probabilities of half-tile h while the value waves consume
//    those of half-tile h - 1.  The value waves, which have the lighter
//    share of the arithmetic, also copy the rows global -> LDS (8 rows
//    each) into three slots of 64 rows, one and a half tiles ahead of use;
//    the slot ids go through a small LDS ring two tiles ahead of that, so
//    that no register is ever the destination of a row or id load in flight.
//    A score wave issues no copies: its only loads are its queries.
//
// Every wait is exact: each wave counts the loads it has issued and records
// the issue index of each operation it will wait for; loads retire in issue
// order, so "at most (issued - 1 - index) outstanding" proves that operation
// complete.  Stores are not counted, which can only make a wait stricter.
//
// The extend instantiation (EXT) serves several query tokens per request: a
// workgroup's 64 rows are (token, head) pairs of one virtual request (a
// request and a block of its query tokens, built on the device: by a pre-pass
// kernel, or for small calls by wave 0 of every workgroup here), a score
// wave's 16 rows belong to one token whose causal limit masks its scores,
// and a token without visible tokens in a piece yields an empty partial
// (lse -inf).
#include "decode_host.h"
#include "extend_common.h"

namespace fp8mla {
namespace {

using namespace decode;

constexpr int NWAVES = 12;
constexpr int THREADS = 64 * NWAVES;              // 768
constexpr int GROUPS = 4;                         // head groups of 16: one per score wave
constexpr int WG_HEADS = GROUPS * HEADS;          // 64
constexpr int TILE = 64;                          // tokens per tile
constexpr int TILE_SHIFT = 6;
constexpr int NSLOTS = 3;                         // row slots (tile j in slot j % 3)
constexpr int ROW_SLOTS = KV_CHUNKS + 1;          // 37 (odd 16-byte stride)
constexpr int ROWB = 16 * ROW_SLOTS;              // 592
constexpr int TILE_BYTES = TILE * ROWB;           // 37888
constexpr int KSTEPS = KV_WIDTH / 64;             // 9
constexpr int QSTEPS = 2 * KSTEPS;                // 18
constexpr int COPIERS = 8;                        // the value waves (which also copy the rows)
constexpr int ROWS_PER_COPIER = TILE / COPIERS;   // 8 rows copied by each value wave
constexpr int DMA_OPS = (ROWS_PER_COPIER * ROW_SLOTS + 63) / 64;  // 5
constexpr int VCOLS = V_WIDTH / COPIERS;          // 64 output columns per value wave
constexpr int VBLOCKS = VCOLS / 16;               // 4 column blocks of 16
static_assert(VBLOCKS == 4, "output stores take the column blocks in two pairs");
constexpr int ID_SLOTS = 4;                       // slot-id ring entries per copying wave
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

// Global -> LDS copy of 4 bytes per active lane (lane l's dword lands at
// lds_base + 4 l), with the wait state an LDS DMA needs after an M0 write.
__device__ __forceinline__ void issue_lds_dma4(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(g), "s"(lds_base)
               : "memory", "m0");
}

// Wait until at most n (wave-uniform) of this wave's vector-memory operations
// are outstanding, rounded down to the counts this pipeline produces (a
// smaller count only waits longer).  n < 0 cannot occur.
__device__ __forceinline__ void wait_vm_atmost(int n) {
  n = __builtin_amdgcn_readfirstlane(n);
  if (n >= 16) wait_vm<16>();
  else if (n >= 11) wait_vm<11>();
  else if (n >= 7) wait_vm<7>();
  else if (n >= 6) wait_vm<6>();
  else if (n >= 5) wait_vm<5>();
  else if (n >= 2) wait_vm<2>();
  else if (n >= 1) wait_vm<1>();
  else wait_vm<0>();
  asm volatile("" ::: "memory");  // no LDS read of landed data moves above the wait
}

template <bool EXT>
__global__ __launch_bounds__(THREADS) void mla_split_h64_kernel(const SplitParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t kv_lds[NSLOTS * TILE_BYTES];
  // slot ids of a tile's rows, per copying wave: [value wave][ring entry][row]
  __shared__ int32_t idring[COPIERS][ID_SLOTS][ROWS_PER_COPIER];
  // probabilities of a half-tile, per head group: [parity][group][block][lane]
  __shared__ uint2 pbuf[2][GROUPS][2][64];
  // rescale factor of each head's running sums at a half-tile: [parity][head][group]
  __shared__ __attribute__((aligned(16))) float abuf[2][HEADS][GROUPS];
  // a finished request's (or piece's) row sums and maxima: [group][head]
  __shared__ float lfin[GROUPS][HEADS];
  __shared__ float mfin[GROUPS][HEADS];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t = lane & 15;
  const int g = lane >> 4;

  // p.HG counts sets of 64 heads here
  int item = blockIdx.x;
  if (p.HG > 1) item = (int)(blockIdx.x & 7) * p.xcd_per + (int)(blockIdx.x >> 3);
  if (item >= p.items) return;
  const int seg = item / p.HG;
  const int hs = item - seg * p.HG;

  if constexpr (EXT) {
    // a small call's list of virtual requests, laid out here by every
    // workgroup (same values) instead of by a pre-pass kernel
    if (p.list.qo_indptr != nullptr) {
      if (w == 0) build_list_wave(p, lane);
      __syncthreads();
    }
  }

  SegmentSpan span;
  // (extend: the virtual requests' CSR counts tiles already)
  if (!find_segment<EXT ? 0 : TILE_SHIFT, THREADS, WG_HEADS, !EXT>(p, seg, hs, lane, span)) return;
  const int ntiles = __builtin_amdgcn_readfirstlane(span.ntiles);
  using Cursor = TileCursor<TILE_SHIFT, EXT>;
  Cursor cc;  // tile being worked on (score waves: scores; value waves: P.V)
  cc.start(p, span, lane);

  // lane index the compiler cannot see through: per-lane address math is
  // redone at each use instead of held in registers across the tile loop
  auto opaque_lane = [&]() -> int {
    int l = lane;
    asm volatile("" : "+v"(l));
    return l;
  };
  // Row tt of head group hg: partial-result row, and (extend) token of the
  // block and head.
  auto group_row = [&](int hg, int tt, int& tok, int& hd) {
    const int r = hs * WG_HEADS + hg * HEADS + tt;
    tok = 0;
    hd = r;
    if constexpr (EXT) {
      if (p.rows_per_tok > 0) {
        tok = (hg * HEADS) / p.rows_per_tok;
        hd = hg * HEADS - tok * p.rows_per_tok + tt;
      }
    }
    return r;
  };

  // ---- loads and their bookkeeping.  nops counts this wave's loads (a
  // score wave: query loads; a value wave: row and id copies); a recorded
  // index i is complete once at most nops - 1 - i loads are outstanding.
  int nops = 0;
  auto wait_done = [&](int op) { wait_vm_atmost(nops - 1 - op); };
  // k loads issued: returns the index of the last (all of it wave-uniform)
  auto count_ops = [&](int k) -> int {
    nops = __builtin_amdgcn_readfirstlane(nops + k);
    return nops - 1;
  };

  bool whole_request = span.j0 == 0;
  int P_cur = span.P0;
  const int H2 = 2 * ntiles;  // intervals with scores; one more for the last P.V

  if (w < GROUPS) {
    // ======================= score wave: head group s ======================
    const int s = w;
    int tk = 0, head = 0;
    group_row(s, t, tk, head);
    // query of head group s, in the d-order of the K reads: step 2i + e,
    // lane (t, g): q[head t][64i + 16g + 8e .. +8]
    auto q_ptr = [&](const Cursor& c) -> const uint16_t* {
      int64_t qrow = c.b;
      if constexpr (EXT) qrow = c.q_row0() + min(tk, c.q_tokens() - 1);
      return p.q + (qrow * p.H + min(head, p.H - 1)) * KV_WIDTH + 16 * g;
    };
    bf16x8_t qr[QSTEPS];
    issue_load_q(qr, q_ptr(cc));
    int q_op = count_ops(QSTEPS);
    wait_done(q_op);
    auto row_idle = [&]() -> bool {
      if constexpr (EXT) return head >= p.H || tk >= cc.q_tokens();
      return head >= p.H;
    };
    // Scores enter the softmax as raw * c (c = sm_scale * scale * log2 e)
    // through one FMA with the exponent's offset, and maxima are taken on the
    // raw sums: both need c > 0.  A negative c is applied by negating the
    // query (exact), c = 0 (every score 0) by a zero query and c taken as 1.
    const float c_in = p.score_scale;
    const float c_mag = c_in > 0.f ? c_in : (c_in < 0.f ? -c_in : 1.0f);
    // the landed query of the current request, made ready for the MFMAs
    auto ready_q = [&]() {
      pin_q(qr);
      if (c_in < 0.f) {
#pragma unroll
        for (int i = 0; i < QSTEPS; ++i) {
          u32x4_t v = __builtin_bit_cast(u32x4_t, qr[i]);
          v ^= 0x80008000u;
          qr[i] = __builtin_bit_cast(bf16x8_t, v);
        }
      }
      if (row_idle() || c_in == 0.f) {
#pragma unroll
        for (int i = 0; i < QSTEPS; ++i) qr[i] = bf16x8_t{};
      }
    };
    ready_q();
    __syncthreads();  // rows of tile 0 published (by the value waves)

    auto record_pieces = [&]() {
      if (hs == 0 && threadIdx.x == 0) {
        const int s0 = span.segment_of(P_cur + START_W);
        const int s1 = span.segment_of(P_cur + START_W + TILE_W * (cc.nt - 1));
        p.req_pieces[cc.b] = make_int2(piece_slot(s0, cc.b == span.b0), s1 - s0 + 1);
      }
    };
    if (whole_request) record_pieces();

    // score operand offsets: block b of half-tile h is tile block 2h + b;
    // lane (t, g) reads chunk 4i + g of its MFMA row t
    const int k_off0 = t * ROWB + 16 * g;                // even block: row t
    const int k_off1 = (16 + (t ^ 12)) * ROWB + 16 * g;  // odd block: row 16 + (t ^ 12)
    const int s_tok0 = 4 * g;                            // tokens of the lane's rows, even block
    const int s_tok1 = 16 + 4 * (g ^ 3);                 // odd block (XOR 12)

    float m_run = -INFINITY;
    float l_w = 0.f;
    bool q_wait = false;  // the next request's query is in flight

    for (int h = 0; h <= H2; ++h) {
      const int m = h >> 1;
      if (h < H2) {
        const int half = h & 1;
        if (q_wait) {
          wait_done(q_op);
          ready_q();
          q_wait = false;
        }
        const int tile_lo = cc.tile_lo();
        int tile_hi = cc.tile_hi();
        if constexpr (EXT) {  // this group's token sees the first lim tokens of the request
          const int len = cc.hi - cc.lo;
          const int lim = p.causal ? len - (cc.q_tokens() - 1 - tk) : len;
          tile_hi = min(tile_hi, cc.lo + max(lim, 0));
        }
        const uint8_t* slot = kv_lds + (m % NSLOTS) * TILE_BYTES + 32 * ROWB * half;
        f32x4_t a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0, c0 = a0, c1 = a0;
        const uint8_t* kp0 = slot + k_off0;
        const uint8_t* kp1 = slot + k_off1;
#pragma unroll
        for (int i = 0; i < KSTEPS; ++i) {
          const u32x4_t kv0 = *reinterpret_cast<const u32x4_t*>(kp0 + 64 * i);
          const u32x4_t kv1 = *reinterpret_cast<const u32x4_t*>(kp1 + 64 * i);
          a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16x8(kv0[0], kv0[1]), qr[2 * i], a0, 0, 0, 0);
          c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16x8(kv1[0], kv1[1]), qr[2 * i], c0, 0, 0, 0);
          a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16x8(kv0[2], kv0[3]), qr[2 * i + 1], a0, 0, 0, 0);
          c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16x8(kv1[2], kv1[3]), qr[2 * i + 1], c0, 0, 0, 0);
        }
        // raw score sums (unscaled); tokens past the end of the request or
        // the causal limit -inf
        float s0[4], s1[4];
        const int hb = tile_lo + 32 * half;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          s0[r] = a0[r];
          s1[r] = c0[r];
        }
        if (hb + 32 > tile_hi) {  // (wave-uniform)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            s0[r] = hb + s_tok0 + r < tile_hi ? s0[r] : -INFINITY;
            s1[r] = hb + s_tok1 + r < tile_hi ? s1[r] : -INFINITY;
          }
        }
        float lmax = max3f(max3f(s0[0], s0[1], s0[2]), max3f(s0[3], s1[0], s1[1]),
                           max3f(s1[2], s1[3], -INFINITY));
        lmax = wave_max_over_groups(lmax) * c_mag;  // over the half-tile's 32 tokens, scaled
        const float m_new = max_f32(m_run, lmax);
        // extend: while a token has seen nothing (m -inf), subtract 0 instead
        const float m_sub = EXT && m_new == -INFINITY ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_sub);
        l_w *= alpha;
        m_run = m_new;
        float pr0[4], pr1[4];
        const float m_p = m_sub - kPScaleLog2;  // probabilities scaled by 2^15 (FP16 P.V)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pr0[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[r], c_mag, -m_p));
          pr1[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[r], c_mag, -m_p));
        }
        const uint32_t p01 = pack_f16x2(pr0[0], pr0[1]), p23 = pack_f16x2(pr0[2], pr0[3]);
        const uint32_t q01 = pack_f16x2(pr1[0], pr1[1]), q23 = pack_f16x2(pr1[2], pr1[3]);
        // the row sums take the probabilities as rounded for P.V
        const f16x2_t one2 = {(_Float16)1.0f, (_Float16)1.0f};
        l_w = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, p01), one2, l_w, false);
        l_w = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, p23), one2, l_w, false);
        l_w = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, q01), one2, l_w, false);
        l_w = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, q23), one2, l_w, false);
        pbuf[h & 1][s][0][lane] = make_uint2(p01, p23);
        pbuf[h & 1][s][1][lane] = make_uint2(q01, q23);
        if (g == 0) abuf[h & 1][t][s] = alpha;

        if (half == 1) {
          const bool last_of_request = cc.j + 1 == cc.nt;
          if (last_of_request || m + 1 == ntiles) {
            // the request's (or piece's) row sums and maximum, for the value waves
            const float lsum = wave_sum_over_groups(l_w);
            if (g == 0) {
              lfin[s][t] = lsum;
              mfin[s][t] = m_run;
            }
            l_w = 0.f;
            m_run = -INFINITY;
          }
          if (last_of_request && m + 1 < ntiles) {
            P_cur += TILE_W * cc.nt + START_W;
            cc.advance(p, lane);
            whole_request = true;
            record_pieces();
            issue_load_q(qr, q_ptr(cc));  // waited for at the start of the next interval
            q_op = count_ops(QSTEPS);
            q_wait = true;
          } else if (m + 1 < ntiles) {
            // (not past the segment's last tile: the cursor would walk the
            // rest of the request list, empty padding included, for nothing)
            cc.advance(p, lane);
          }
        }
      }
      __syncthreads();
    }
  } else {
    // ======================= value wave: columns 64v .. +63 ====================
    const int v = w - GROUPS;
    Cursor lc = cc;  // next tile whose slot ids are copied
    const uint32_t lds_tiles = (uint32_t)(uintptr_t)(
        (__attribute__((address_space(3))) uint8_t*)&kv_lds[0]);
    const uint32_t lds_ids = (uint32_t)(uintptr_t)(
        (__attribute__((address_space(3))) int32_t*)&idring[v][0][0]);
    // slot ids of the load cursor's tile j: lane r < 8 copies the id of row
    // 8v + r into ring entry j % 4 (tokens past the request: the tile's
    // first row; past the segment's last tile: entry 0 of kv_indices, unused,
    // and the cursor stays on the last tile rather than walk the rest of the
    // request list)
    auto copy_ids = [&](int j) -> int {
      const int ln = opaque_lane();
      const uint32_t base =
          __builtin_amdgcn_readfirstlane(lds_ids + 4 * ROWS_PER_COPIER * (j & (ID_SLOTS - 1)));
      const int tlo = lc.tile_lo();
      const int tok = tlo + ROWS_PER_COPIER * v + ln;
      const int32_t* a =
          j < ntiles && lc.nt > 0 ? p.indices + (tok < lc.tile_hi() ? tok : tlo) : p.indices;
      if (ln < ROWS_PER_COPIER) issue_lds_dma4(a, base);
      if (j + 1 < ntiles) lc.advance(p, lane);
      return count_ops(1);
    };
    // rows 8v .. 8v+7 of tile j into slot j % 3: op i fills 16-byte LDS
    // chunks 64i .. 64i+63 of the wave's block of 8 x 37 (row P / 37, chunk
    // P % 37; the pad chunk gets a copy of chunk 35; lanes past the block
    // masked off).  What a lane copies depends on the tile only through the
    // row's slot id, so the rest is computed once: per op, the byte offset
    // of the lane's row id in a ring entry and the address of its chunk in
    // row 0 of the pool (held opaque, so that it stays in registers).
    uint32_t rof[DMA_OPS];
    uint64_t cbase[DMA_OPS];
#pragma unroll
    for (int i = 0; i < DMA_OPS; ++i) {
      const int P = 64 * i + lane;
      const int r = P / ROW_SLOTS;
      const int c = min(P - r * ROW_SLOTS, KV_CHUNKS - 1);
      rof[i] = 4u * (uint32_t)(r & (ROWS_PER_COPIER - 1));
      cbase[i] = (uint64_t)(uintptr_t)(p.pool + 16 * c);
      asm volatile("" : "+v"(rof[i]), "+v"(cbase[i]));
    }
    // Its slot ids must have landed.  Returns the index of its last op.
    auto copy_rows = [&](int j) -> int {
      const uint32_t base = __builtin_amdgcn_readfirstlane(
          lds_tiles + (uint32_t)((j % NSLOTS) * TILE_BYTES + ROWS_PER_COPIER * v * ROWB));
      const uint8_t* ids = reinterpret_cast<const uint8_t*>(&idring[v][j & (ID_SLOTS - 1)][0]);
      // every op's slot id first, so that the LDS reads overlap (a copy's
      // asm clobbers memory: no read can move past it)
      uint32_t sid[DMA_OPS];
#pragma unroll
      for (int i = 0; i < DMA_OPS; ++i) sid[i] = *reinterpret_cast<const uint32_t*>(ids + rof[i]);
      const int ln = opaque_lane();
#pragma unroll
      for (int i = 0; i < DMA_OPS; ++i) {
        const uint32_t s = sid[i];  // negative ids compare as large
        const uint8_t* a = reinterpret_cast<const uint8_t*>(
            (uintptr_t)(cbase[i] + (uint64_t)(s < p.max_slot ? s : p.max_slot) * KV_WIDTH));
        if (i < DMA_OPS - 1 || ln < ROWS_PER_COPIER * ROW_SLOTS - 64 * (DMA_OPS - 1)) {
          // decode reads each row once per head set, close together in time
          // (non-temporal hint); extend re-reads a request's rows for each of
          // its query blocks (default policy)
          if constexpr (!EXT) issue_lds_dma16_nt(a, base + 1024 * i);
          else issue_lds_dma16(a, base + 1024 * i);
        }
      }
      return count_ops(DMA_OPS);
    };

    // Prologue: slot ids of tiles 0-3; once those of 0 and 1 have landed,
    // rows of tiles 0 and 1.  Pipeline state for the first odd interval
    // (m = 0): rows of tile m + 1 and ids of tiles m + 2, m + 3 in flight.
    copy_ids(0);
    const int id1 = copy_ids(1);
    int id_a = copy_ids(2);  // ids of tile m + 2
    int id_b = copy_ids(3);  // ids of tile m + 3
    wait_done(id1);
    const int r0 = copy_rows(0);
    int r_m1 = ntiles > 1 ? copy_rows(1) : -1;  // last op of the rows of tile m + 1
    wait_done(r0);
    __syncthreads();  // rows of tile 0 published

    // Odd interval 2m + 1.  At its start (after the barrier that ends the
    // last reads of tile m - 1, this role's P.V of its second half) the rows
    // of tile m + 2 go into tile m - 1's slot and the ids of tile m + 4 into
    // the ring entry of tile m's; at its end the rows of tile m + 1 (read
    // from the next interval on) are waited for, and the barrier that ends
    // the interval publishes them to the score waves.
    int r_new = -1, id_new = -1;
    auto issue_copies = [&](int m) {
      r_new = -1;
      if (m + 2 < ntiles) {
        wait_done(id_a);  // ids of tile m + 2
        r_new = copy_rows(m + 2);
      }
      id_new = copy_ids(m + 4);
    };
    auto wait_copies = [&]() {
      wait_done(r_m1);
      r_m1 = r_new;
      id_a = id_b;
      id_b = id_new;
    };

    // transposed value reads: for the 32 tokens of a half-tile, lane i of
    // group g supplies row 4g + i/2 (i/2 < 4: even block rows 4g..4g+3) or
    // row 16 + 4(g^3) + i/2 - 4 (odd block rows (4g..4g+3)^12): exactly the
    // tokens whose probabilities lane (t, g) of a score wave produced
    auto tr_offset = [&]() -> int {
      const int ln = opaque_lane();
      const int tt = ln & 15, gg = ln >> 4;
      const int row = (tt >> 1) < 4 ? 4 * gg + (tt >> 1) : 16 + 4 * (gg ^ 3) + (tt >> 1) - 4;
      return row * ROWB + 8 * (tt & 1) + VCOLS * v;
    };

    f32x4_t O[GROUPS][VBLOCKS];
#pragma unroll
    for (int hg = 0; hg < GROUPS; ++hg)
#pragma unroll
      for (int c = 0; c < VBLOCKS; ++c) O[hg][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto finish_request = [&](bool complete) {
      // lane (t, g) holds columns 64v + 16c + 4g + 0..3 of head t of every
      // group; lanes g and g ^ 1 pair them up for 16-byte stores (pair_blocks)
      const int ln = opaque_lane();
      const int tt = ln & 15, gg = ln >> 4;
      const int col = VCOLS * v + paired_col(gg);  // + 32 k for block pair k
#pragma unroll
      for (int hg = 0; hg < GROUPS; ++hg) {
        const float l = lfin[hg][tt];
        int tok_g, head_g;
        const int row_g = group_row(hg, tt, tok_g, head_g);
        bool idle = head_g >= p.H;
        if constexpr (EXT) idle = idle || tok_g >= cc.q_tokens();
        if (complete) {
          // extend: a token with no visible token gets a zero row
          const float inv = EXT && l == 0.f ? 0.f : p.kv_scale / l;
          uint4 d[2];
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const f32x4_t& a = O[hg][2 * k];
            const f32x4_t& b = O[hg][2 * k + 1];
            d[k] = pair_blocks(make_uint2(pack_bf16x2(a[0] * inv, a[1] * inv),
                                          pack_bf16x2(a[2] * inv, a[3] * inv)),
                               make_uint2(pack_bf16x2(b[0] * inv, b[1] * inv),
                                          pack_bf16x2(b[2] * inv, b[3] * inv)));
          }
          if (!idle) {
            int64_t orow = cc.b;
            if constexpr (EXT) orow = cc.q_row0() + tok_g;
            uint16_t* op = p.out + (orow * p.H + head_g) * V_WIDTH + col;
            *reinterpret_cast<uint4*>(op) = d[0];
            *reinterpret_cast<uint4*>(op + 32) = d[1];
          }
        } else {
          const int64_t piece = (int64_t)piece_slot(seg, cc.b == span.b0) * p.Hp + row_g;
          const bool empty = EXT && l == 0.f;  // extend: no visible token in this piece
          const float inv = empty ? 0.f : 1.0f / l;
          uint16_t* op = p.part_o + piece * V_WIDTH + col;
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const f32x4_t& a = O[hg][2 * k];
            const f32x4_t& b = O[hg][2 * k + 1];
            *reinterpret_cast<uint4*>(op + 32 * k) =
                pair_blocks(make_uint2(pack_f16x2(a[0] * inv, a[1] * inv),
                                       pack_f16x2(a[2] * inv, a[3] * inv)),
                            make_uint2(pack_f16x2(b[0] * inv, b[1] * inv),
                                       pack_f16x2(b[2] * inv, b[3] * inv)));
          }
          if (v == hg && gg == 0)
            p.part_lse[piece] = empty ? -INFINITY : mfin[hg][tt] + __builtin_amdgcn_logf(l) - kPScaleLog2;
        }
      }
#pragma unroll
      for (int hg = 0; hg < GROUPS; ++hg)
#pragma unroll
        for (int c = 0; c < VBLOCKS; ++c) O[hg][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    };

    for (int h = 0; h <= H2; ++h) {
      if (h & 1) issue_copies(h >> 1);
      if (h >= 1) {
        // P.V of half-tile h - 1: tile pm, half ph
        const int hp = h - 1;
        const int pm = hp >> 1, ph = hp & 1;
        const int ln = opaque_lane();
        // rescale a head group's sums only where one of its maxima moved
        // (the four groups' factors of a head in one read)
        const f32x4_t alpha = *reinterpret_cast<const f32x4_t*>(&abuf[hp & 1][ln & 15][0]);
#pragma unroll
        for (int hg = 0; hg < GROUPS; ++hg) {
          if (__ballot(alpha[hg] != 1.0f)) {
#pragma unroll
            for (int c = 0; c < VBLOCKS; ++c) O[hg][c] *= alpha[hg];
          }
        }
        f16x8_t pb[GROUPS];
#pragma unroll
        for (int hg = 0; hg < GROUPS; ++hg) {
          const uint2 x = pbuf[hp & 1][hg][0][ln];
          const uint2 y = pbuf[hp & 1][hg][1][ln];
          const u32x4_t pv = {x.x, x.y, y.x, y.y};
          pb[hg] = __builtin_bit_cast(f16x8_t, pv);
        }
        // Rows past the request's end in a partial tile are copies of the
        // tile's first row with probability 0, so their value bytes need no
        // masking.
        const uint8_t* vb = kv_lds + (pm % NSLOTS) * TILE_BYTES + 32 * ROWB * ph + tr_offset();
        // the half-tile's transposed reads, conversions and 16 MFMAs, in the
        // compiler's order (with three waves per SIMD, pinning the groups in
        // order measured 1% slower)
        i32x2_t vt[VBLOCKS];
#pragma unroll
        for (int c = 0; c < VBLOCKS; ++c)
          vt[c] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (__attribute__((address_space(3))) i32x2_t*)(vb + 16 * c));
        f16x8_t va[VBLOCKS];
#pragma unroll
        for (int c = 0; c < VBLOCKS; ++c) va[c] = e4m3x8_to_f16x8((uint32_t)vt[c].x, (uint32_t)vt[c].y);
#pragma unroll
        for (int c = 0; c < VBLOCKS; ++c)
#pragma unroll
          for (int hg = 0; hg < GROUPS; ++hg)
            O[hg][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va[c], pb[hg], O[hg][c], 0, 0, 0);
        if (ph == 1) {
          const bool last_of_request = cc.j + 1 == cc.nt;
          if (last_of_request || pm + 1 == ntiles) finish_request(whole_request && last_of_request);
          if (last_of_request && pm + 1 < ntiles) whole_request = true;
          if (pm + 1 < ntiles) cc.advance(p, lane);
        }
      }
      if (h & 1) wait_copies();
      __syncthreads();
    }
  }
  wait_vm<0>();  // retire loads issued past the last tile
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
