// Virtual requests of an extend call (internal): a request and a block of up
// to T of its query tokens, the unit the 64-row split kernel works on.  The
// arithmetic that lays them out is shared by the pre-pass kernel (any size)
// and by the split kernel itself, which builds the list in one wave per
// workgroup when the call is small enough (kFusedListMaxBatch requests,
// kFusedListMaxVirtual list entries) to save the pre-pass launch.
#pragma once

#include "decode_common.h"
#include "launch.h"

namespace fp8mla {
namespace decode {

// Calls the split kernel lays out itself: one request per lane, four
// 64-entry chunks of the list.
constexpr int kFusedListMaxBatch = 64;
constexpr int kFusedListMaxVirtual = 256;

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// Request b's query rows [q_lo, q_hi) and kv_indices range [kv_lo, kv_hi),
// each indptr entry clamped into its array so that no access leaves it.
struct RequestRanges {
  int q_lo, q_hi, kv_lo, kv_hi;
};
__device__ __forceinline__ RequestRanges request_ranges(const int32_t* qo, const int32_t* kv, int b,
                                                        int total_q, int total_kv) {
  RequestRanges r;
  r.q_lo = clampi(qo[b], 0, total_q);
  r.q_hi = max(r.q_lo, clampi(qo[b + 1], 0, total_q));
  r.kv_lo = clampi(kv[b], 0, total_kv);
  r.kv_hi = max(r.kv_lo, clampi(kv[b + 1], 0, total_kv));
  return r;
}

// The block of query tokens i0 .. of a request: it reads the first `len`
// tokens of the request's list (its last token's limit under the causal
// mask, the whole list without), i.e. `ntiles` 64-token tiles, the last
// holding `tail` tokens; its rows start at query row q_row.
struct VirtualRequest {
  int ntiles, tail, kv_lo, q_row, ntok;
};
__device__ __forceinline__ VirtualRequest virtual_request(const RequestRanges& r, int i0, int T,
                                                          bool causal, int total_q) {
  constexpr int TS = kExtendTileShift;
  VirtualRequest vr;
  const int ql = r.q_hi - r.q_lo;
  const int kl = r.kv_hi - r.kv_lo;
  // (the clamps only act on a non-monotone indptr: they keep every query row
  // the split kernel touches inside [0, total_q))
  vr.ntok = min(clampi(ql - i0, 1, T), total_q);
  const int len = causal ? clampi(kl - ql + i0 + vr.ntok, 0, kl) : kl;
  vr.ntiles = (len >> TS) + ((len & ((1 << TS) - 1)) != 0);
  vr.tail = len - (vr.ntiles > 0 ? (vr.ntiles - 1) << TS : 0);  // tokens of the last tile, 1 .. 64
  vr.kv_lo = r.kv_lo;
  vr.q_row = clampi(r.q_lo + i0, 0, total_q - vr.ntok);
  return vr;
}
__device__ __forceinline__ int2 vinfo_of(const VirtualRequest& vr) {
  return make_int2(vr.kv_lo, vr.q_row | ((vr.ntok - 1) << kExtTokShift) |
                                 ((vr.ntiles > 0 ? vr.tail - 1 : 0) << kExtTailShift));
}

// The list of a small call, built by one wave (every lane, lane = request,
// then lane = list entry in chunks of 64): the same vindptr [vmax + 1],
// vinfo [vmax] and header {V, CSR total} as the pre-pass kernel, entries
// V .. vmax - 1 empty, and every entry empty when the CSR total passes
// kExtendMaxTiles (an index array that breaks the call's contract).  Each
// workgroup of the split kernel writes the same values; every entry is
// written once, from registers, so that a workgroup reading an entry sees
// that value whichever workgroup wrote it last.
__device__ __forceinline__ void build_list_wave(const SplitParams& p, int lane) {
  const ExtendList& e = p.list;
  const int vmax = p.B;
  int nblk = 0;
  RequestRanges r{0, 0, 0, 0};
  if (lane < e.batch) {
    r = request_ranges(e.qo_indptr, e.kv_indptr, lane, e.total_q, e.total_kv);
    nblk = (r.q_hi - r.q_lo + e.T - 1) / e.T;
  }
  const int incl = wave_inclusive_scan(nblk, lane);
  const int first = min(incl - nblk, vmax);  // this request's first list entry
  const int V = min(__builtin_amdgcn_readlane(incl, 63), vmax);
  constexpr int CHUNKS = kFusedListMaxVirtual / 64;
  int ntiles[CHUNKS];
  int2 vi[CHUNKS];
  int pos[CHUNKS];
  int64_t total = 0;
#pragma unroll
  for (int k = 0; k < CHUNKS; ++k) {
    const int v = 64 * k + lane;
    ntiles[k] = 0;
    vi[k] = make_int2(0, 0);
    if (64 * k < V) {  // (wave-uniform)
      // its request: the last b with first_b <= v
      int b = 0;
      for (int c = 1; c < e.batch; ++c) b = __builtin_amdgcn_readlane(first, c) <= v ? c : b;
      RequestRanges rb;
      rb.q_lo = __shfl(r.q_lo, b);
      rb.q_hi = __shfl(r.q_hi, b);
      rb.kv_lo = __shfl(r.kv_lo, b);
      rb.kv_hi = __shfl(r.kv_hi, b);
      const int fb = __shfl(first, b);
      if (v < V) {
        const VirtualRequest vr = virtual_request(rb, (v - fb) * e.T, e.T, p.causal != 0, e.total_q);
        ntiles[k] = vr.ntiles;
        vi[k] = vinfo_of(vr);
      }
    }
    const int inc = wave_inclusive_scan(ntiles[k], lane);
    pos[k] = (int)min(total + inc - ntiles[k], kExtendMaxTiles);
    total += __builtin_amdgcn_readlane(inc, 63);
  }
  const bool fits = total <= kExtendMaxTiles;
#pragma unroll
  for (int k = 0; k < CHUNKS; ++k) {
    const int v = 64 * k + lane;
    if (v < vmax) {
      e.indptr_out[v] = !fits ? 0 : (v < V ? pos[k] : (int32_t)total);
      e.vinfo_out[v] = v < V ? vi[k] : make_int2(0, 0);
    }
  }
  if (lane == 0) {
    e.indptr_out[vmax] = fits ? (int32_t)total : 0;
    e.hdr[0] = V;
    e.hdr[1] = fits ? (int32_t)total : 0;
  }
}

}  // namespace decode
}  // namespace fp8mla
