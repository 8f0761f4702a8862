// Internal host-side launch interface between the C ABI (api.cpp) and the
// kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fp8mla {

hipError_t launch_cast_pool(const uint8_t* pool, int64_t num_slots, uint16_t* out,
                            hipStream_t stream, int num_cus);

hipError_t launch_gather_cast(const uint8_t* pool, int64_t num_slots, const int32_t* indices,
                              int64_t n, uint16_t* out, hipStream_t stream,
                              int num_cus);

hipError_t launch_scatter_cast(const uint16_t* src, int64_t src_row_stride, int64_t n,
                               const int32_t* slots, uint8_t* pool, int64_t num_slots,
                               float inv_scale, bool saturate, hipStream_t stream);

// Decode schedule: equal segments of the request-tile list x head groups, and the split-K
// workspace layout (per-request piece ranges, partial outputs, log2-sum-exp values).
// Which split kernel a decode call runs: FP8 rows with 16 heads per
// workgroup, FP8 rows with 64 heads per workgroup (64 or more heads), or
// BF16 rows.
enum class DecodeKernel { kFp8, kFp8H64, kBf16 };

// FP8 calls with at least this many heads use the 64-head workgroups, when
// there is enough work for them: at least kH64MinTilesPerCu 64-token tiles
// per workgroup slot (CUs / head sets).  With fewer tokens the 16-head
// kernel, which has four times as many workgroups per segment, exposes more
// parallelism.
constexpr int kH64MinHeads = 64;
constexpr int kH64MinTilesPerCu = 4;

struct DecodePlan {
  DecodeKernel kernel;
  int32_t HG;          // head groups (of 16, or of 64 for kFp8H64)
  int32_t Hp;          // padded head count = HG * heads per workgroup
  int32_t nseg;        // segments the list of request tiles is cut into
  int32_t items;       // nseg * HG workgroups doing work
  int32_t xcd_per;     // work items per XCD slot of the launch grid
  int32_t grid;        // launched workgroups (>= items)
  size_t part_o_offset;  // byte offset of the partial outputs inside the workspace
  size_t lse_offset;   // byte offset of the lse array inside the workspace
  size_t workspace_bytes;
};

// max_segments > 0 bounds the number of segments (for tests of split
// invariance and for tuning); the workspace size does not depend on it.
DecodePlan plan_mla_decode(int32_t batch, int32_t num_heads, int64_t total_tokens, int num_cus,
                           DecodeKernel kernel, int32_t max_segments = 0);

inline DecodeKernel fp8_decode_kernel(int32_t num_heads, int64_t total_tokens, int num_cus) {
  if (num_heads < kH64MinHeads) return DecodeKernel::kFp8;
  const int64_t head_sets = (num_heads + 63) / 64;
  const int64_t tiles = (total_tokens + 63) / 64;
  return tiles >= (int64_t)kH64MinTilesPerCu * num_cus / head_sets ? DecodeKernel::kFp8H64
                                                                  : DecodeKernel::kFp8;
}

hipError_t launch_mla_decode(const uint16_t* q, const uint8_t* kv_pool, int64_t num_slots,
                             const int32_t* kv_indptr, const int32_t* kv_indices,
                             int64_t total_tokens, int32_t batch, int32_t num_heads, float scale,
                             float sm_scale, uint16_t* out, void* workspace, const DecodePlan& plan,
                             hipStream_t stream);

hipError_t launch_mla_decode_bf16(const uint16_t* q, const uint16_t* kv, int64_t num_rows,
                                  const int32_t* kv_indptr, const int32_t* kv_indices,
                                  int64_t total_tokens, int32_t batch, int32_t num_heads,
                                  float scale, float sm_scale, uint16_t* out, void* workspace,
                                  const DecodePlan& plan, hipStream_t stream);

hipError_t launch_mla_decode_h64(const uint16_t* q, const uint8_t* kv_pool, int64_t num_slots,
                                 const int32_t* kv_indptr, const int32_t* kv_indices,
                                 int64_t total_tokens, int32_t batch, int32_t num_heads,
                                 float scale, float sm_scale, uint16_t* out, void* workspace,
                                 const DecodePlan& plan, hipStream_t stream);

// Extend: several query tokens per request, causal or not.  The 64-row
// kernel runs over virtual requests -- a request and a block of T of its
// query tokens -- that a one-workgroup pre-pass builds on the device from
// qo_indptr and kv_indptr, so the host never reads either.  Rows of a
// workgroup are (token, head) pairs: T = 64 / rows_per_tok tokens of
// rows_per_tok rows (heads rounded up to 16) when that is at most 64, else
// one token and HG sets of 64 heads.
struct ExtendPlan {
  int32_t rows_per_tok;   // 0 when heads > 64
  int32_t tokens_per_wg;  // T
  int32_t HG;
  int32_t Hp;             // partial-result rows per virtual request (64 * HG)
  int32_t vmax;           // bound on the virtual requests: batch + ceil(total_q / T)
  int32_t nseg;
  int32_t items;
  int32_t xcd_per;
  int32_t grid;
  size_t vstart_offset;   // int32 [batch + 1]: first virtual request of each request
  size_t vindptr_offset;  // int32 [vmax + 1]: CSR of the tiles each virtual request reads
  size_t vinfo_offset;    // int2 [vmax]
  size_t pieces_offset;   // int2 [vmax]: (segment of the first piece, pieces)
  size_t part_o_offset;   // fp16 [2 * nseg * Hp * 512]: two piece slots per segment
  size_t lse_offset;      // float [2 * nseg * Hp]
  size_t workspace_bytes; // also holds the header {virtual requests, CSR total} at offset 0
};

// Limits of an extend call.  Query rows pack into 23 bits of the virtual
// requests' info.  The virtual requests' CSR counts 64-token tiles and must
// stay within kExtendMaxTiles, so that the split's int32 weights (4 per
// tile, 6 per request) cannot overflow; the host checks a bound of that
// total computed from the sizes alone (extend_tile_bound).
constexpr int64_t kExtendMaxQueryRows = (int64_t)1 << 23;
constexpr int64_t kExtendMaxTiles = (int64_t)1 << 28;
constexpr int64_t kExtendMaxVirtual = (int64_t)1 << 25;
constexpr int kExtendTileShift = 6;  // the 64-row kernel's tile: 64 tokens

// Upper bound on the tiles of the virtual requests of any extend call with
// these sizes whose indptr arrays satisfy the contract: request b's
// ceil(q_b / T) blocks each see at most kv_b tokens, so the tokens seen sum
// to at most (ceil(total_q / T) + 1) * total_kv, and every block adds at
// most one partial tile.
int64_t extend_tile_bound(int32_t batch, int32_t num_heads, int64_t total_q, int64_t total_kv);

ExtendPlan plan_mla_extend(int32_t batch, int32_t num_heads, int64_t total_q, int num_cus);

hipError_t launch_mla_extend(const uint16_t* q, const uint8_t* kv_pool, int64_t num_slots,
                             const int32_t* qo_indptr, const int32_t* kv_indptr,
                             const int32_t* kv_indices, int64_t total_q, int64_t total_kv,
                             int32_t batch, int32_t num_heads, float scale, float sm_scale,
                             bool causal, uint16_t* out, void* workspace, const ExtendPlan& plan,
                             hipStream_t stream);

// Contract check of a request CSR and its slot ids (status int32[4], see
// fp8mla_check_indices); indptr or indices may be NULL to skip that part.
hipError_t launch_index_check(const int32_t* indptr, int32_t batch, int64_t total,
                              const int32_t* indices, int64_t num_slots, int32_t* status,
                              bool reset, int num_cus, hipStream_t stream);

// HBM ceiling probes (benchmark-only).
hipError_t launch_probe_read(const void* src, int64_t bytes, int grid, int unroll, uint32_t* sink,
                             hipStream_t stream);
hipError_t launch_probe_copy12(const void* src, int64_t bytes, void* dst, int grid, int unroll,
                               hipStream_t stream);
hipError_t launch_probe_write(void* dst, int64_t bytes, int grid, int unroll, hipStream_t stream);
hipError_t launch_probe_gather(const uint8_t* pool, int64_t num_slots, const int32_t* idx,
                               int64_t n, int grid, int chunks_in_flight, uint32_t* sink,
                               hipStream_t stream);

constexpr int kFp8TileTokens = 128;
constexpr int kH64TileTokens = 64;
constexpr int kBf16TileTokens = 64;

}  // namespace fp8mla
