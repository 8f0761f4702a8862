// Split-K MLA decode over BF16 latent rows, for gfx950: the attention that
// follows a cast on the pages' fallback paths ("The Gather-Then-Cast Pivot",
// Reasoning Process: gather the active rows, cast them to BF16, run the
// attention over indices 0..n-1; "The KV Cache Cast Bottleneck", The
// Context: cast the whole pool, run the attention with the original
// indices).  Benchmark-only: it exists so that those paths can be timed end
// to end against the fused FP8 kernel.
//
// Same computation as the FP8 kernel with K[t, :] = scale * kv[slot_t, :]
// read as BF16 (1152-byte rows), the same work split over 64-token request
// tiles, the same partial format and the same combine kernel.  Inside a
// workgroup (4 waves, 16 heads), per tile:
//  * the tile's 64 rows are copied global -> LDS (global_load_lds, 16 bytes
//    per lane) one tile ahead, into one of two slots of 64 x 1168 bytes
//    (72 data chunks + 1 pad: an odd 16-byte stride, so the row reads of 16
//    lanes hit distinct banks);
//  * wave w scores tokens [16w, 16w+16): S^T = K q^T, MFMA 16x16x32 bf16,
//    K read with ds_read_b128 (lane (t, g) reads dims 32s + 8g .. +8 of row t
//    in step s), q held in registers in the same order;
//  * the softmax is exchanged through LDS as in the FP8 kernel;
//  * wave w owns output columns [128w, 128w + 128) of O^T = V^T P^T (MFMA
//    16x16x32 f16, 8 column blocks), reading the transposed value operand
//    with ds_read_b64_tr_b16 and converting it to FP16; the probabilities
//    are FP16 scaled by 2^15, as in the FP8 kernels, so that values of
//    opposite sign up to 448 that cancel keep their rounding error inside
//    the tolerance (BF16 probabilities, 8 significant bits, do not).
// Rows must hold values within the fp16 range (|v| <= 65504) for the value
// operand and the partials; BF16 values of that range convert to FP16
// exactly down to 2^-17 in magnitude.  The rows produced by the casts hold
// E4M3 values (|v| <= 448, exact in FP16).
#include "decode_host.h"

namespace fp8mla {
namespace {

using namespace decode;

typedef __attribute__((ext_vector_type(4))) short i16x4_t;

// Two BF16 values (low half first) to two FP16 values: exact for BF16
// values within the FP16 range down to 2^-17 in magnitude, rounded to
// nearest below.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  return pack_f16x2(__builtin_bit_cast(float, w << 16), __builtin_bit_cast(float, w & 0xFFFF0000u));
}

constexpr int NWAVES = 4;
constexpr int THREADS = 64 * NWAVES;             // 256
constexpr int TILE = 16 * NWAVES;                // 64 tokens per tile
constexpr int TILE_SHIFT = 6;
constexpr int ROW_BYTES = 2 * KV_WIDTH;          // 1152
constexpr int ROW_CHUNKS = ROW_BYTES / 16;       // 72
constexpr int ROW_SLOTS = ROW_CHUNKS + 1;        // 73: one pad chunk, odd stride
constexpr int ROWB = 16 * ROW_SLOTS;             // 1168
constexpr int TILE_BYTES = TILE * ROWB;          // 74752
constexpr int QSTEPS = KV_WIDTH / 32;            // 18 MFMA steps of 32 dims
constexpr int DMA_OPS = (16 * ROW_SLOTS + 63) / 64;  // 19 copy ops per wave per tile
constexpr int VBLOCKS = V_WIDTH / NWAVES / 16;   // 8 output blocks of 16 columns per wave
static_assert(TILE == 1 << TILE_SHIFT, "tile size");
static_assert(TILE == kBf16TileTokens, "host and kernel tile sizes agree");

__global__ __launch_bounds__(THREADS) void mla_split_bf16_kernel(const SplitParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t kv_lds[2 * TILE_BYTES];
  __shared__ float mx_lds[NWAVES][HEADS];
  __shared__ uint2 p_lds[NWAVES][64];
  __shared__ float l_lds[NWAVES][HEADS];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t = lane & 15;
  const int g = lane >> 4;

  int item = blockIdx.x;
  if (p.HG > 1) item = (int)(blockIdx.x & 7) * p.xcd_per + (int)(blockIdx.x >> 3);
  if (item >= p.items) return;
  const int seg = item / p.HG;
  const int hg = item - seg * p.HG;
  const int head = hg * HEADS + t;

  SegmentSpan span;
  if (!find_segment<TILE_SHIFT, THREADS>(p, seg, hg, lane, span)) return;
  const int ntiles = span.ntiles;
  TileCursor<TILE_SHIFT> cc;
  cc.start(p, span, lane);
  TileCursor<TILE_SHIFT> lc = cc;

  // index of the load cursor's tile (lane r < 16 and its copies: token
  // 16w + r; tokens past the request read the tile's first row), then advance
  auto load_next_index = [&]() -> int32_t {
    const int tlo = lc.tile_lo();
    const int tok = tlo + 16 * w + t;
    const int32_t* a = lc.nt > 0 ? p.indices + (tok < lc.tile_hi() ? tok : tlo) : p.indices;
    const int32_t v = issue_load_i32(a);
    lc.advance(p, lane);
    return v;
  };
  const uint32_t lds_tiles = (uint32_t)(uintptr_t)(
      (__attribute__((address_space(3))) uint8_t*)&kv_lds[0]);
  // rows 16w .. 16w+15 of tile k into slot k & 1: op j fills 16-byte LDS
  // chunks 64j .. 64j+63 of the wave's block of 16 x 73 (row P / 73, chunk
  // P % 73; the pad chunk gets a copy of chunk 71; lanes past the block in
  // the last op are masked off)
  auto issue_tile = [&](int k, int32_t idx) {
    const uint32_t base =
        __builtin_amdgcn_readfirstlane(lds_tiles + (uint32_t)((k & 1) * TILE_BYTES + 16 * w * ROWB));
#pragma unroll
    for (int j = 0; j < DMA_OPS; ++j) {
      const int P = 64 * j + lane;
      const int r = P / ROW_SLOTS;
      const int c = min(P - r * ROW_SLOTS, ROW_CHUNKS - 1);
      const uint32_t s = (uint32_t)__shfl(idx, r & 15);
      const uint8_t* a = p.pool + (uint64_t)(s < p.max_slot ? s : p.max_slot) * ROW_BYTES + 16 * c;
      if (j < DMA_OPS - 1 || P < 16 * ROW_SLOTS) issue_lds_dma16(a, base + 1024 * j);
    }
  };

  // query: lane (t, g) holds q[head t][32s + 8g .. +8] for step s (compiler
  // loads; waited for with the tile's own wait)
  bf16x8_t qr[QSTEPS];
  auto load_query = [&](int b) {
    const uint16_t* qp = p.q + ((int64_t)b * p.H + min(head, p.H - 1)) * KV_WIDTH + 8 * g;
#pragma unroll
    for (int s = 0; s < QSTEPS; ++s) qr[s] = *reinterpret_cast<const bf16x8_t*>(qp + 32 * s);
  };
  auto zero_pad_heads = [&]() {
    if (head >= p.H) {
#pragma unroll
      for (int s = 0; s < QSTEPS; ++s) qr[s] = bf16x8_t{};
    }
  };

  // Prologue: index of tile 0, rows of tile 0, index of tile 1, query.
  int32_t ix = load_next_index();
  wait_vm<0>();
  pin(ix);
  issue_tile(0, ix);
  ix = load_next_index();
  load_query(cc.b);
  wait_vm<0>();
  pin(ix);
  zero_pad_heads();
  __syncthreads();

  f32x4_t O[VBLOCKS];
#pragma unroll
  for (int c = 0; c < VBLOCKS; ++c) O[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;
  float l_w = 0.f;
  bool whole_request = span.j0 == 0;
  int P_cur = span.P0;
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
    // lane (t, g) holds columns 128w + 16c + 4g + 0..3 of head t; lanes g and
    // g ^ 1 pair them up for 16-byte stores (pair_blocks)
    const int col = 128 * w + paired_col(g);  // + 32 k for block pair k
    if (complete) {
      const float inv = p.kv_scale / l;
      uint4 d[VBLOCKS / 2];
#pragma unroll
      for (int k = 0; k < VBLOCKS / 2; ++k)
        d[k] = pair_blocks(make_uint2(pack_bf16x2(O[2 * k][0] * inv, O[2 * k][1] * inv),
                                      pack_bf16x2(O[2 * k][2] * inv, O[2 * k][3] * inv)),
                           make_uint2(pack_bf16x2(O[2 * k + 1][0] * inv, O[2 * k + 1][1] * inv),
                                      pack_bf16x2(O[2 * k + 1][2] * inv, O[2 * k + 1][3] * inv)));
      if (head < p.H) {
        uint16_t* op = p.out + ((int64_t)cc.b * p.H + head) * V_WIDTH + col;
#pragma unroll
        for (int k = 0; k < VBLOCKS / 2; ++k) *reinterpret_cast<uint4*>(op + 32 * k) = d[k];
      }
    } else {
      const int64_t piece = (int64_t)piece_slot(seg, cc.b == span.b0) * p.Hp + head;
      const float inv = 1.0f / l;
      uint16_t* op = p.part_o + piece * V_WIDTH + col;
#pragma unroll
      for (int k = 0; k < VBLOCKS / 2; ++k)
        *reinterpret_cast<uint4*>(op + 32 * k) =
            pair_blocks(make_uint2(pack_f16x2(O[2 * k][0] * inv, O[2 * k][1] * inv),
                                   pack_f16x2(O[2 * k][2] * inv, O[2 * k][3] * inv)),
                        make_uint2(pack_f16x2(O[2 * k + 1][0] * inv, O[2 * k + 1][1] * inv),
                                   pack_f16x2(O[2 * k + 1][2] * inv, O[2 * k + 1][3] * inv)));
      if (w == 0 && g == 0) p.part_lse[piece] = m_run + __builtin_amdgcn_logf(l) - kPScaleLog2;
    }
#pragma unroll
    for (int c = 0; c < VBLOCKS; ++c) O[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    l_w = 0.f;
    m_run = -INFINITY;
  };

  // transposed value reads: supplier lane L = 16g' + 4r + q provides row
  // 32st + 8g' + 4h + r, columns 4q .. 4q+3 of a 16-column block; the
  // receiving lane (t, g) then holds V[32st + 8g + 4h + r][block + t] for
  // r = 0..3 -- A operand elements 8g + 4h + r of row t
  const int tr_off = (8 * g + ((lane >> 2) & 3)) * ROWB + 8 * (lane & 3);

  for (int k = 0; k < ntiles; ++k) {
    const int tile_lo = cc.tile_lo();
    const int tile_hi = cc.tile_hi();
    const bool last_of_request = cc.j + 1 == cc.nt;
    const uint8_t* slot = kv_lds + (k & 1) * TILE_BYTES;
    // next tile's rows into the other slot (free since the last barrier),
    // then the index of the tile after it
    if (k + 1 < ntiles) issue_tile(k + 1, ix);
    ix = load_next_index();

    f32x4_t a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
    const uint8_t* kp = slot + (16 * w + t) * ROWB + 16 * g;
#pragma unroll
    for (int s = 0; s < QSTEPS; s += 2) {
      a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8_t*>(kp + 64 * s),
                                                   qr[s], a0, 0, 0, 0);
      a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8_t*>(kp + 64 * s + 64),
                                                   qr[s + 1], a1, 0, 0, 0);
    }
    float sc[4];
    float lmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool ok = tile_lo + 16 * w + 4 * g + r < tile_hi;
      sc[r] = ok ? (a0[r] + a1[r]) * p.score_scale : -INFINITY;
      lmax = fmaxf(lmax, sc[r]);
    }
    lmax = wave_max_over_groups(lmax);
    if (g == 0) mx_lds[w][t] = lmax;
    __syncthreads();
    float tmax = mx_lds[0][t];
#pragma unroll
    for (int v = 1; v < NWAVES; ++v) tmax = fmaxf(tmax, mx_lds[v][t]);
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    if (__ballot(alpha != 1.0f)) {
#pragma unroll
      for (int c = 0; c < VBLOCKS; ++c) O[c] *= alpha;
      l_w *= alpha;
    }
    m_run = m_new;
    float pr[4];
    const float m_p = m_new - kPScaleLog2;  // probabilities scaled by 2^15 (FP16 P.V)
#pragma unroll
    for (int r = 0; r < 4; ++r) pr[r] = __builtin_amdgcn_exp2f(sc[r] - m_p);
    const uint32_t p01 = pack_f16x2(pr[0], pr[1]);
    const uint32_t p23 = pack_f16x2(pr[2], pr[3]);
    l_w += (f16_lo(p01) + f16_hi(p01)) + (f16_lo(p23) + f16_hi(p23));
    p_lds[w][lane] = make_uint2(p01, p23);
    __syncthreads();

#pragma unroll
    for (int st = 0; st < 2; ++st) {
      // B operand: lane (t, g) holds P[head t][tokens 32st + 8g .. +8]:
      // wave 2st + g/2, its groups 2(g%2) and 2(g%2)+1
      const uint2 x = p_lds[2 * st + (g >> 1)][32 * (g & 1) + t];
      const uint2 y = p_lds[2 * st + (g >> 1)][32 * (g & 1) + 16 + t];
      const u32x4_t pv = {x.x, x.y, y.x, y.y};
      const f16x8_t pb = __builtin_bit_cast(f16x8_t, pv);
      const uint8_t* vb = slot + 32 * st * ROWB + tr_off + 2 * (128 * w);
#pragma unroll
      for (int c = 0; c < VBLOCKS; ++c) {
        const i32x2_t lo = __builtin_bit_cast(i32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4_t*)(vb + 32 * c)));
        const i32x2_t hi = __builtin_bit_cast(i32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4_t*)(vb + 4 * ROWB + 32 * c)));
        const u32x4_t a = {bf16x2_to_f16x2((uint32_t)lo.x), bf16x2_to_f16x2((uint32_t)lo.y),
                           bf16x2_to_f16x2((uint32_t)hi.x), bf16x2_to_f16x2((uint32_t)hi.y)};
        O[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), pb, O[c], 0, 0, 0);
      }
    }

    if (last_of_request || k + 1 == ntiles) finish_request(whole_request && last_of_request);
    const bool new_q = last_of_request && k + 1 < ntiles;
    if (new_q) {
      P_cur += TILE_W * cc.nt + START_W;
      cc.advance(p, lane);
      whole_request = true;
      record_pieces();
      load_query(cc.b);
    } else {
      cc.advance(p, lane);
    }
    // everything issued in this tile has landed: rows of tile k+1, the next
    // index, a new query
    wait_vm<0>();
    pin(ix);
    if (new_q) zero_pad_heads();
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_mla_decode_bf16(const uint16_t* q, const uint16_t* kv, int64_t num_rows,
                                  const int32_t* kv_indptr, const int32_t* kv_indices,
                                  int64_t total_tokens, int32_t batch, int32_t num_heads,
                                  float scale, float sm_scale, uint16_t* out, void* workspace,
                                  const DecodePlan& pl, hipStream_t stream) {
  const decode::SplitParams sp = make_split_params(q, kv, num_rows, kv_indptr, kv_indices,
                                                   total_tokens, batch, num_heads, scale,
                                                   sm_scale, out, workspace, pl);
  hipLaunchKernelGGL(mla_split_bf16_kernel, dim3(pl.grid), dim3(THREADS), 0, stream, sp);
  hipError_t e = hipGetLastError();
  // no tokens, or one segment (every request complete in it): nothing to merge
  if (e != hipSuccess || total_tokens == 0 || pl.nseg == 1) return e;
  return launch_mla_combine(sp, stream);
}

}  // namespace fp8mla
