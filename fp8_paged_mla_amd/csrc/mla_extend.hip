// MLA extend (prefill) attention over the paged FP8-E4M3FN latent cache, for
// gfx950: several new query tokens per request, with a causal mask over the
// request's cache list.  This is the extend path of "When a Faster Kernel
// Doesn't Speed Up Serving" (Step 3, CastFromFP8: the prefill attention
// reads the request's whole history, which the original stack first casts to
// BF16); here the FP8 rows are read and dequantised in the kernel, as on the
// decode path.
//
// Query token i of request b sees the first n_i tokens of the request's
// cache list: n_i = kv_len - q_len + i + 1 with the mask (the new tokens are
// the list's last q_len entries), kv_len without.
//
// Three kernels on the caller's stream, no host reads of the index arrays:
//  1. extend_prepass_kernel (one workgroup) cuts every request's query
//     tokens into blocks of T and lays the blocks out as virtual requests:
//     a block reads the first n tokens of its request's list, n being its
//     last token's limit; their CSR in 64-token tiles, and per block its
//     first kv_indices entry, first query row and the tokens of its last
//     tile.  Calls of at most 64 requests and 256 list entries skip it: the
//     split kernel builds the same list itself (extend_common.h).
//  2. mla_split_h64_kernel<true> runs the 64-row split kernel over them: a
//     block's T tokens x H heads share every KV tile, each 16-row group
//     masked by its own token's limit.
//  3. extend_combine_kernel merges the partials of blocks that span
//     segments, and writes the zero rows of empty blocks.
#include "decode_host.h"
#include "extend_common.h"

namespace fp8mla {
namespace {

using namespace decode;

constexpr int PRE_THREADS = 1024;
constexpr int PRE_WAVES = PRE_THREADS / 64;
constexpr int COMBINE_ROWS = 4;  // rows per combine workgroup, one wave each

__device__ __forceinline__ int64_t shfl_up_i64(int64_t x, int o) {
  const int lo = __shfl_up((int)(uint32_t)x, o);
  const int hi = __shfl_up((int)(x >> 32), o);
  return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// Exclusive prefix sum of x over the workgroup's 1024 lanes; `total` gets the
// sum.  All lanes must call it.
__device__ __forceinline__ int64_t block_exclusive_scan(int64_t x, int64_t& total) {
  __shared__ int64_t wave_sums[PRE_WAVES];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  int64_t inc = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t y = shfl_up_i64(inc, o);
    if (lane >= o) inc += y;
  }
  if (lane == 63) wave_sums[w] = inc;
  __syncthreads();
  if (w == 0) {
    int64_t s = lane < PRE_WAVES ? wave_sums[lane] : 0;
#pragma unroll
    for (int o = 1; o < PRE_WAVES; o <<= 1) {
      const int64_t y = shfl_up_i64(s, o);
      if (lane >= o) s += y;
    }
    if (lane < PRE_WAVES) wave_sums[lane] = s;
  }
  __syncthreads();
  const int64_t base = w > 0 ? wave_sums[w - 1] : 0;
  total = wave_sums[PRE_WAVES - 1];
  __syncthreads();  // wave_sums is rewritten by the next call
  return base + inc - x;
}

// hdr = {virtual requests V, CSR total}; vstart [B + 1]; vindptr [vmax + 1]
// and vinfo [vmax], entries V.. padded as empty requests, so that the split
// kernel can walk all vmax of them without reading V.  V is capped at vmax
// and the CSR total at kExtendMaxTiles; both caps are reached only by index
// arrays that break the call's contract (non-monotone indptr), and then
// every virtual request is made empty: the combine writes zero rows and no
// read leaves its array.
__global__ __launch_bounds__(PRE_THREADS) void extend_prepass_kernel(
    const int32_t* __restrict__ qo_indptr, const int32_t* __restrict__ kv_indptr, int32_t B,
    int32_t total_q, int32_t total_kv, int32_t T, int32_t causal, int32_t vmax,
    int32_t* __restrict__ hdr, int32_t* __restrict__ vstart, int32_t* __restrict__ vindptr,
    int2* __restrict__ vinfo) {
  // blocks per request -> first virtual request of each request
  int64_t carry = 0;
  for (int c = 0; c < B; c += PRE_THREADS) {
    const int b = c + (int)threadIdx.x;
    int nblk = 0;
    if (b < B) {
      const RequestRanges r = request_ranges(qo_indptr, kv_indptr, b, total_q, total_kv);
      nblk = (r.q_hi - r.q_lo + T - 1) / T;
    }
    int64_t tot;
    const int64_t ex = block_exclusive_scan(nblk, tot);
    if (b < B) vstart[b] = (int32_t)min(carry + ex, (int64_t)vmax);
    carry += tot;
  }
  const int V = (int)min(carry, (int64_t)vmax);
  if (threadIdx.x == 0) vstart[B] = V;
  __syncthreads();

  // per virtual request: its request (the last b with vstart[b] <= v), its
  // token block, the tokens it reads, and the CSR of their tiles
  int64_t ncarry = 0;
  for (int c = 0; c < V; c += PRE_THREADS) {
    const int v = c + (int)threadIdx.x;
    int ntiles = 0;
    int2 vi = make_int2(0, 0);
    if (v < V) {
      int lo = 0, hi = B - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (vstart[mid] <= v) lo = mid;
        else hi = mid - 1;
      }
      const RequestRanges r = request_ranges(qo_indptr, kv_indptr, lo, total_q, total_kv);
      const VirtualRequest vr = virtual_request(r, (v - vstart[lo]) * T, T, causal != 0, total_q);
      ntiles = vr.ntiles;
      vi = vinfo_of(vr);
    }
    int64_t tot;
    const int64_t pos = ncarry + block_exclusive_scan(ntiles, tot);
    if (v < V) {
      vindptr[v] = (int32_t)min(pos, kExtendMaxTiles);
      vinfo[v] = vi;
    }
    ncarry += tot;
  }
  const bool fits = ncarry <= kExtendMaxTiles;
  for (int v = V + (int)threadIdx.x; v <= vmax; v += PRE_THREADS) {
    vindptr[v] = fits ? (int32_t)ncarry : 0;
    if (v < vmax) vinfo[v] = make_int2(0, 0);
  }
  if (!fits) {  // the split kernel sees only empty requests
    __syncthreads();
    for (int v = (int)threadIdx.x; v < V; v += PRE_THREADS) vindptr[v] = 0;
  }
  if (threadIdx.x == 0) {
    hdr[0] = V;
    hdr[1] = fits ? (int32_t)ncarry : 0;
  }
}

struct ExtendCombineParams {
  const int32_t* hdr;
  const int2* vinfo;
  const int2* pieces;
  const uint16_t* part_o;
  const float* part_lse;
  uint16_t* out;
  int32_t H;
  int32_t Hp;
  int32_t rows_per_tok;
  float kv_scale;
};

// One wave per (virtual request, row).  Blocks whose request lies within one
// segment were written by the split kernel (one piece); blocks that read no
// token get zero rows; the rest merge their pieces.
__global__ __launch_bounds__(64 * COMBINE_ROWS) void extend_combine_kernel(const ExtendCombineParams p) {
  const int v = blockIdx.x;
  // The count, the block's vinfo and its piece range are loaded together (one
  // memory latency): vinfo and pieces hold vmax = gridDim.x entries, so the
  // reads are in bounds for every block; past the count they are not used.
  const int count = p.hdr[0];
  const int2 vi = p.vinfo[v];
  const int2 rp = p.pieces[v];
  asm volatile("" ::"s"(count), "s"(vi.x), "s"(vi.y), "s"(rp.x), "s"(rp.y));  // all three issued here
  if (v >= count) return;
  const int row = blockIdx.y * COMBINE_ROWS + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  int tk = 0, head = row;
  if (p.rows_per_tok > 0) {
    tk = row / p.rows_per_tok;
    head = row - tk * p.rows_per_tok;
  }
  if (head >= p.H || tk > ((vi.y >> kExtTokShift) & 3)) return;
  if (rp.y == 1) return;
  uint16_t* op = p.out + ((int64_t)((vi.y & kExtQ0Mask) + tk) * p.H + head) * V_WIDTH;
  if (rp.y == 0) {
    *reinterpret_cast<uint4*>(op + 8 * lane) = make_uint4(0u, 0u, 0u, 0u);
    return;
  }
  merge_pieces(p.part_o, p.part_lse, p.Hp, rp.x, rp.y, row, p.kv_scale, op, lane);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

int64_t extend_tile_bound(int32_t batch, int32_t num_heads, int64_t total_q, int64_t total_kv) {
  const int rows = (num_heads + 15) / 16 * 16;
  const int64_t T = rows <= 64 ? 64 / rows : 1;
  const int64_t blocks = (total_q + T - 1) / T;
  const int64_t vmax = (int64_t)batch + blocks;
  const int64_t tiles_of_kv = (total_kv + (1 << kExtendTileShift) - 1) >> kExtendTileShift;
  // (blocks + 1) * tiles_of_kv cannot overflow: blocks < 2^23, tiles_of_kv < 2^25
  return (blocks + 1) * tiles_of_kv + vmax;
}

ExtendPlan plan_mla_extend(int32_t batch, int32_t num_heads, int64_t total_q, int num_cus) {
  ExtendPlan pl{};
  const int rows = (num_heads + 15) / 16 * 16;
  if (rows <= 64) {
    pl.rows_per_tok = rows;
    pl.tokens_per_wg = 64 / rows;
    pl.HG = 1;
  } else {
    pl.rows_per_tok = 0;
    pl.tokens_per_wg = 1;
    pl.HG = (rows + 63) / 64;
  }
  pl.Hp = 64 * pl.HG;
  const int64_t vmax = (int64_t)batch + (total_q + pl.tokens_per_wg - 1) / pl.tokens_per_wg;
  pl.vmax = (int32_t)(vmax < INT32_MAX ? vmax : INT32_MAX);
  int32_t nseg = num_cus / pl.HG;
  pl.nseg = nseg < 1 ? 1 : nseg;
  pl.items = pl.nseg * pl.HG;
  if (pl.HG > 1) {
    pl.xcd_per = (pl.items + 7) / 8;
    pl.grid = 8 * pl.xcd_per;
  } else {
    pl.xcd_per = pl.items;
    pl.grid = pl.items;
  }
  const size_t V = (size_t)pl.vmax;
  size_t off = 256;  // header
  pl.vstart_offset = off;
  off = align256(off + 4 * ((size_t)batch + 1));
  pl.vindptr_offset = off;
  off = align256(off + 4 * (V + 1));
  pl.vinfo_offset = off;
  off = align256(off + 8 * V);
  pl.pieces_offset = off;
  off = align256(off + 8 * V);
  pl.part_o_offset = off;
  off = align256(off + 2 * (2 * (size_t)pl.nseg) * pl.Hp * V_WIDTH);  // two piece slots per segment
  pl.lse_offset = off;
  off = align256(off + 4 * (2 * (size_t)pl.nseg) * pl.Hp);
  pl.workspace_bytes = off;
  return pl;
}

hipError_t launch_mla_extend(const uint16_t* q, const uint8_t* kv_pool, int64_t num_slots,
                             const int32_t* qo_indptr, const int32_t* kv_indptr,
                             const int32_t* kv_indices, int64_t total_q, int64_t total_kv,
                             int32_t batch, int32_t num_heads, float scale, float sm_scale,
                             bool causal, uint16_t* out, void* workspace, const ExtendPlan& pl,
                             hipStream_t stream) {
  if (total_q == 0) return hipSuccess;
  char* ws = reinterpret_cast<char*>(workspace);
  int32_t* hdr = reinterpret_cast<int32_t*>(ws);
  int32_t* vstart = reinterpret_cast<int32_t*>(ws + pl.vstart_offset);
  int32_t* vindptr = reinterpret_cast<int32_t*>(ws + pl.vindptr_offset);
  int2* vinfo = reinterpret_cast<int2*>(ws + pl.vinfo_offset);
  int2* pieces = reinterpret_cast<int2*>(ws + pl.pieces_offset);
  // small calls: the split kernel lays out the list itself (one wave per
  // workgroup), which saves the pre-pass launch
  const bool fused_list = batch <= decode::kFusedListMaxBatch && pl.vmax <= decode::kFusedListMaxVirtual;
  hipError_t e = hipSuccess;
  if (!fused_list) {
    hipLaunchKernelGGL(extend_prepass_kernel, dim3(1), dim3(PRE_THREADS), 0, stream, qo_indptr,
                       kv_indptr, batch, (int32_t)total_q, (int32_t)total_kv, pl.tokens_per_wg,
                       causal ? 1 : 0, pl.vmax, hdr, vstart, vindptr, vinfo);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }

  decode::SplitParams sp{};
  sp.q = q;
  sp.pool = kv_pool;
  sp.indptr = vindptr;
  sp.indices = kv_indices;
  sp.out = out;
  sp.part_o = reinterpret_cast<uint16_t*>(ws + pl.part_o_offset);
  sp.part_lse = reinterpret_cast<float*>(ws + pl.lse_offset);
  sp.req_pieces = pieces;
  sp.max_slot = num_slots > 0 ? (uint32_t)(num_slots - 1) : 0u;
  sp.total_tokens = (int32_t)kExtendMaxTiles;  // bound of the tile CSR (clamps only)
  sp.B = pl.vmax;  // V real virtual requests, then empty ones
  sp.H = num_heads;
  sp.HG = pl.HG;
  sp.Hp = pl.Hp;
  sp.nseg = pl.nseg;
  sp.items = pl.items;
  sp.xcd_per = pl.xcd_per;
  sp.score_scale = (float)((double)sm_scale * (double)scale * 1.4426950408889634);
  sp.kv_scale = scale;
  sp.vinfo = vinfo;
  sp.rows_per_tok = pl.rows_per_tok;
  sp.causal = causal ? 1 : 0;
  if (fused_list) {
    sp.list.qo_indptr = qo_indptr;
    sp.list.kv_indptr = kv_indptr;
    sp.list.indptr_out = vindptr;
    sp.list.vinfo_out = vinfo;
    sp.list.hdr = hdr;
    sp.list.batch = batch;
    sp.list.total_q = (int32_t)total_q;
    sp.list.total_kv = (int32_t)total_kv;
    sp.list.T = pl.tokens_per_wg;
  }
  e = launch_mla_split_h64_extend(sp, pl.grid, stream);
  if (e != hipSuccess) return e;

  ExtendCombineParams cp;
  cp.hdr = hdr;
  cp.vinfo = vinfo;
  cp.pieces = pieces;
  cp.part_o = sp.part_o;
  cp.part_lse = sp.part_lse;
  cp.out = out;
  cp.H = num_heads;
  cp.Hp = pl.Hp;
  cp.rows_per_tok = pl.rows_per_tok;
  cp.kv_scale = scale;
  hipLaunchKernelGGL(extend_combine_kernel, dim3(pl.vmax, pl.Hp / COMBINE_ROWS),
                     dim3(64 * COMBINE_ROWS), 0, stream, cp);
  return hipGetLastError();
}

}  // namespace fp8mla
