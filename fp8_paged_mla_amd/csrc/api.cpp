// C ABI of libfp8mla.so: argument validation and dispatch.  Every check runs
// on the host before any HIP call, so a rejected call touches no device.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "../../include/fp8mla.h"
#include "launch.h"

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_num_cus[kMaxDevices];

// Compute units of the current device (cached per device), or -1 on error.
int current_device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
  if (dev < kMaxDevices) {
    const int cached = g_num_cus[dev].load(std::memory_order_relaxed);
    if (cached > 0) return cached;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return -1;
  if (dev < kMaxDevices) g_num_cus[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

constexpr int64_t kMaxSlots = (int64_t)UINT32_MAX;  // slot ids are 32-bit
constexpr int64_t kMaxTokens = (int64_t)INT32_MAX;  // kv_indptr is int32

// Checks shared by the decode entry points (everything but the workspace).
int check_decode_fp8_args(const uint16_t* q, const uint8_t* kv_pool, int64_t num_slots,
                          const int32_t* kv_indptr, const int32_t* kv_indices,
                          int64_t total_tokens, int32_t batch, int32_t num_heads, float scale,
                          float sm_scale, const uint16_t* out) {
  if (batch < 1 || batch > FP8MLA_MAX_BATCH || num_heads < 1 || num_heads > FP8MLA_MAX_HEADS ||
      total_tokens < 0 || total_tokens > kMaxTokens || num_slots < 0 || num_slots > kMaxSlots)
    return FP8MLA_ERR_BAD_SHAPE;
  if (total_tokens > 0 && num_slots == 0) return FP8MLA_ERR_BAD_SHAPE;
  if (!isfinite(scale) || !(scale > 0.0f) || !isfinite(sm_scale)) return FP8MLA_ERR_BAD_SCALAR;
  if (!q || !kv_indptr || !out) return FP8MLA_ERR_NULL_PTR;
  if (total_tokens > 0 && (!kv_pool || !kv_indices)) return FP8MLA_ERR_NULL_PTR;
  if (!aligned16(q) || !aligned16(out) || !aligned4(kv_indptr)) return FP8MLA_ERR_MISALIGNED;
  if (total_tokens > 0 && (!aligned16(kv_pool) || !aligned4(kv_indices)))
    return FP8MLA_ERR_MISALIGNED;
  return FP8MLA_OK;
}

// Split-K scratch of mla_decode_fp8_noalloc, for callers that cannot
// allocate: one array per device, held by every GPU the library runs on
// until the process ends, shared by all such calls on that GPU (they race
// if they overlap).  The decode needs no initialised scratch: every word a
// kernel reads was written earlier in the same call.  On the host `scratch`
// is only a stand-in for the device variable, never a device address: host
// code uses the address hipGetSymbolAddress returns for the current device.
constexpr size_t kScratchBytes = FP8MLA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;

// Device address of the current device's scratch array, looked up once per
// device with that device current; NULL on failure.
void* current_device_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr) return ptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  ptr = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (!ptr) {
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev].store(ptr, std::memory_order_release);
  }
  return ptr;
}

#ifdef FP8MLA_DEBUG_CHECKS
// Debug build: every reading call first runs the index-contract check into
// this sticky per-device status (flags, first bad request, first bad slot
// position, bad slot count), read and cleared by fp8mla_debug_status.  Host
// code uses the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(16) int32_t debug_status[4] = {0, INT32_MAX, INT32_MAX, 0};
std::atomic<int32_t*> g_debug_status_ptr[kMaxDevices];

int32_t* current_device_debug_status() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  int32_t* ptr = g_debug_status_ptr[dev].load(std::memory_order_acquire);
  if (ptr) return ptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  ptr = g_debug_status_ptr[dev].load(std::memory_order_relaxed);
  if (!ptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(debug_status)) != hipSuccess || !p) return nullptr;
    ptr = static_cast<int32_t*>(p);
    g_debug_status_ptr[dev].store(ptr, std::memory_order_release);
  }
  return ptr;
}

hipError_t debug_check(const int32_t* indptr, int32_t batch, int64_t total, const int32_t* indices,
                       int64_t num_slots, int cus, void* stream) {
  int32_t* st = current_device_debug_status();
  if (!st) return hipErrorInvalidSymbol;
  return fp8mla::launch_index_check(indptr, batch, total, indices, num_slots, st, false, cus,
                                    static_cast<hipStream_t>(stream));
}
#else
// Release build: no checks on the reading calls' path.
hipError_t debug_check(const int32_t*, int32_t, int64_t, const int32_t*, int64_t, int, void*) {
  return hipSuccess;
}
#endif

// Sizes an extend call accepts: every count in range, the virtual requests
// and the tile bound of their CSR within what the kernels address.
bool extend_sizes_ok(int32_t batch, int32_t num_heads, int64_t total_q, int64_t total_kv) {
  if (batch < 1 || num_heads < 1 || num_heads > FP8MLA_MAX_HEADS || total_q < 0 ||
      total_q >= fp8mla::kExtendMaxQueryRows || total_kv < 0 || total_kv > kMaxTokens)
    return false;
  if (total_q * num_heads > (int64_t)INT32_MAX) return false;  // query rows
  const int rows = (num_heads + 15) / 16 * 16;
  const int64_t T = rows <= 64 ? 64 / rows : 1;
  if ((int64_t)batch + (total_q + T - 1) / T > fp8mla::kExtendMaxVirtual) return false;
  return fp8mla::extend_tile_bound(batch, num_heads, total_q, total_kv) <= fp8mla::kExtendMaxTiles;
}

}  // namespace

extern "C" {

int fp8mla_abi_version(void) { return 1; }

const char* fp8mla_status_string(int status) {
  switch (status) {
    case FP8MLA_OK: return "ok";
    case FP8MLA_ERR_NULL_PTR: return "a required pointer is NULL";
    case FP8MLA_ERR_BAD_SHAPE: return "invalid size argument";
    case FP8MLA_ERR_MISALIGNED: return "tensor pointer not 16-byte aligned";
    case FP8MLA_ERR_WORKSPACE: return "workspace missing or too small";
    case FP8MLA_ERR_BAD_SCALAR: return "scale / inv_scale must be finite and > 0, sm_scale finite";
    case FP8MLA_ERR_HIP: return "HIP runtime error or kernel launch failure";
    case FP8MLA_ERR_NOT_DEBUG: return "not the debug build (no accumulated check status)";
    default: return "unknown status";
  }
}

int fp8mla_check_indices(const int32_t* indptr, int32_t batch, int64_t total,
                         const int32_t* indices, int64_t num_slots, int32_t* status,
                         void* stream) {
  if (total < 0 || total > kMaxTokens || (indptr && (batch < 1 || batch == INT32_MAX)) ||
      (indices && (num_slots < 1 || num_slots > kMaxSlots)))
    return FP8MLA_ERR_BAD_SHAPE;
  if (!status) return FP8MLA_ERR_NULL_PTR;
  if (!aligned4(status) || (indptr && !aligned4(indptr)) || (indices && !aligned4(indices)))
    return FP8MLA_ERR_MISALIGNED;
  const int cus = current_device_cus();
  if (cus <= 0) return FP8MLA_ERR_HIP;
  const hipError_t e = fp8mla::launch_index_check(indptr, batch, total, indices, num_slots, status,
                                                  true, cus, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8MLA_OK : FP8MLA_ERR_HIP;
}

int fp8mla_debug_status(int32_t* status_out, int32_t reset) {
#ifdef FP8MLA_DEBUG_CHECKS
  if (!status_out) return FP8MLA_ERR_NULL_PTR;
  int32_t* st = current_device_debug_status();
  if (!st) return FP8MLA_ERR_HIP;
  if (hipDeviceSynchronize() != hipSuccess) return FP8MLA_ERR_HIP;
  if (hipMemcpy(status_out, st, 4 * sizeof(int32_t), hipMemcpyDeviceToHost) != hipSuccess)
    return FP8MLA_ERR_HIP;
  if (reset) {
    const int32_t init[4] = {0, INT32_MAX, INT32_MAX, 0};
    if (hipMemcpy(st, init, sizeof(init), hipMemcpyHostToDevice) != hipSuccess) return FP8MLA_ERR_HIP;
  }
  return FP8MLA_OK;
#else
  (void)status_out;
  (void)reset;
  return FP8MLA_ERR_NOT_DEBUG;
#endif
}

int cast_pool_fp8_bf16(const uint8_t* pool, int64_t num_slots, uint16_t* out, void* stream) {
  if (num_slots < 0 || num_slots > kMaxSlots) return FP8MLA_ERR_BAD_SHAPE;
  if (num_slots == 0) return FP8MLA_OK;
  if (!pool || !out) return FP8MLA_ERR_NULL_PTR;
  if (!aligned16(pool) || !aligned16(out)) return FP8MLA_ERR_MISALIGNED;
  const int cus = current_device_cus();
  if (cus <= 0) return FP8MLA_ERR_HIP;
  const hipError_t e =
      fp8mla::launch_cast_pool(pool, num_slots, out, static_cast<hipStream_t>(stream), cus);
  return e == hipSuccess ? FP8MLA_OK : FP8MLA_ERR_HIP;
}

int gather_cast_fp8_bf16(const uint8_t* pool, int64_t num_slots, const int32_t* indices,
                         int64_t n, uint16_t* out, void* stream) {
  if (n < 0 || n > kMaxTokens || num_slots < 0 || num_slots > kMaxSlots)
    return FP8MLA_ERR_BAD_SHAPE;
  if (n == 0) return FP8MLA_OK;
  if (num_slots == 0) return FP8MLA_ERR_BAD_SHAPE;
  if (!pool || !indices || !out) return FP8MLA_ERR_NULL_PTR;
  if (!aligned16(pool) || !aligned16(out) || !aligned4(indices)) return FP8MLA_ERR_MISALIGNED;
  const int cus = current_device_cus();
  if (cus <= 0) return FP8MLA_ERR_HIP;
  if (debug_check(nullptr, 0, n, indices, num_slots, cus, stream) != hipSuccess)
    return FP8MLA_ERR_HIP;
  const hipError_t e = fp8mla::launch_gather_cast(pool, num_slots, indices, n, out,
                                                  static_cast<hipStream_t>(stream), cus);
  return e == hipSuccess ? FP8MLA_OK : FP8MLA_ERR_HIP;
}

int scatter_cast_bf16_fp8(const uint16_t* src, int64_t n, int64_t src_row_stride,
                          const int32_t* slots, uint8_t* pool, int64_t num_slots,
                          float inv_scale, int32_t saturate, void* stream) {
  if (n < 0 || n > kMaxTokens || num_slots < 0 || num_slots > kMaxSlots)
    return FP8MLA_ERR_BAD_SHAPE;
  if (src_row_stride < FP8MLA_KV_WIDTH || src_row_stride % 8 != 0 ||
      src_row_stride > (int64_t)1 << 40)
    return FP8MLA_ERR_BAD_SHAPE;
  if (!isfinite(inv_scale) || !(inv_scale > 0.0f)) return FP8MLA_ERR_BAD_SCALAR;
  if (n == 0) return FP8MLA_OK;
  if (num_slots == 0) return FP8MLA_ERR_BAD_SHAPE;
  if (!src || !slots || !pool) return FP8MLA_ERR_NULL_PTR;
  if (!aligned16(src) || !aligned16(pool) || !aligned4(slots)) return FP8MLA_ERR_MISALIGNED;
  // int32 slot ids name at most INT32_MAX slots; negative ids then compare as
  // unsigned values past the last slot and are skipped.
  const int64_t writable = num_slots < (int64_t)INT32_MAX ? num_slots : (int64_t)INT32_MAX;
  const hipError_t e = fp8mla::launch_scatter_cast(src, src_row_stride, n, slots, pool, writable,
                                                   inv_scale, saturate != 0,
                                                   static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8MLA_OK : FP8MLA_ERR_HIP;
}

size_t mla_extend_fp8_workspace_bytes(int32_t batch, int32_t num_heads, int64_t total_q) {
  if (!extend_sizes_ok(batch, num_heads, total_q, 0) || total_q == 0) return 0;
  const int cus = current_device_cus();
  if (cus <= 0) return 0;
  return fp8mla::plan_mla_extend(batch, num_heads, total_q, cus).workspace_bytes;
}

int mla_extend_fp8(const uint16_t* q, const uint8_t* kv_pool, int64_t num_slots,
                   const int32_t* qo_indptr, const int32_t* kv_indptr, const int32_t* kv_indices,
                   int64_t total_q, int64_t total_kv, int32_t batch, int32_t num_heads,
                   float scale, float sm_scale, int32_t causal, uint16_t* out, void* workspace,
                   size_t workspace_bytes, void* stream) {
  if (!extend_sizes_ok(batch, num_heads, total_q, total_kv) || num_slots < 0 ||
      num_slots > kMaxSlots)
    return FP8MLA_ERR_BAD_SHAPE;
  if (total_kv > 0 && num_slots == 0) return FP8MLA_ERR_BAD_SHAPE;
  if (!isfinite(scale) || !(scale > 0.0f) || !isfinite(sm_scale)) return FP8MLA_ERR_BAD_SCALAR;
  if (total_q == 0) return FP8MLA_OK;
  if (!q || !qo_indptr || !kv_indptr || !out || !workspace) return FP8MLA_ERR_NULL_PTR;
  if (total_kv > 0 && (!kv_pool || !kv_indices)) return FP8MLA_ERR_NULL_PTR;
  if (!aligned16(q) || !aligned16(out) || !aligned4(qo_indptr) || !aligned4(kv_indptr) ||
      !aligned16(workspace))
    return FP8MLA_ERR_MISALIGNED;
  if (total_kv > 0 && (!aligned16(kv_pool) || !aligned4(kv_indices))) return FP8MLA_ERR_MISALIGNED;
  const int cus = current_device_cus();
  if (cus <= 0) return FP8MLA_ERR_HIP;
  const fp8mla::ExtendPlan plan = fp8mla::plan_mla_extend(batch, num_heads, total_q, cus);
  if (workspace_bytes < plan.workspace_bytes) return FP8MLA_ERR_WORKSPACE;
  if (debug_check(qo_indptr, batch, total_q, nullptr, 0, cus, stream) != hipSuccess ||
      debug_check(kv_indptr, batch, total_kv, kv_indices, num_slots, cus, stream) != hipSuccess)
    return FP8MLA_ERR_HIP;
  const hipError_t e = fp8mla::launch_mla_extend(q, kv_pool, num_slots, qo_indptr, kv_indptr,
                                                 kv_indices, total_q, total_kv, batch, num_heads,
                                                 scale, sm_scale, causal != 0, out, workspace,
                                                 plan, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8MLA_OK : FP8MLA_ERR_HIP;
}

size_t mla_decode_fp8_workspace_bytes(int32_t batch, int32_t num_heads, int64_t total_tokens) {
  if (batch < 1 || batch > FP8MLA_MAX_BATCH || num_heads < 1 || num_heads > FP8MLA_MAX_HEADS ||
      total_tokens < 0 || total_tokens > kMaxTokens)
    return 0;
  if (total_tokens == 0) return 0;
  const int cus = current_device_cus();
  if (cus <= 0) return 0;
  return fp8mla::plan_mla_decode(batch, num_heads, total_tokens, cus,
                                 fp8mla::fp8_decode_kernel(num_heads, total_tokens, cus))
      .workspace_bytes;
}

int mla_decode_fp8(const uint16_t* q, const uint8_t* kv_pool, int64_t num_slots,
                   const int32_t* kv_indptr, const int32_t* kv_indices, int64_t total_tokens,
                   int32_t batch, int32_t num_heads, float scale, float sm_scale, uint16_t* out,
                   void* workspace, size_t workspace_bytes, void* stream) {
  return mla_decode_fp8_segments(q, kv_pool, num_slots, kv_indptr, kv_indices, total_tokens,
                                 batch, num_heads, scale, sm_scale, out, workspace,
                                 workspace_bytes, INT32_MAX, stream);
}

int mla_decode_fp8_segments(const uint16_t* q, const uint8_t* kv_pool, int64_t num_slots,
                            const int32_t* kv_indptr, const int32_t* kv_indices,
                            int64_t total_tokens, int32_t batch, int32_t num_heads, float scale,
                            float sm_scale, uint16_t* out, void* workspace,
                            size_t workspace_bytes, int32_t num_segments, void* stream) {
  const int st = check_decode_fp8_args(q, kv_pool, num_slots, kv_indptr, kv_indices, total_tokens,
                                       batch, num_heads, scale, sm_scale, out);
  if (st != FP8MLA_OK) return st;
  if (num_segments < 1) return FP8MLA_ERR_BAD_SHAPE;
  if (total_tokens > 0 && !workspace) return FP8MLA_ERR_NULL_PTR;
  if (total_tokens > 0 && !aligned16(workspace)) return FP8MLA_ERR_MISALIGNED;
  const int cus = current_device_cus();
  if (cus <= 0) return FP8MLA_ERR_HIP;
  const fp8mla::DecodePlan plan = fp8mla::plan_mla_decode(
      batch, num_heads, total_tokens, cus, fp8mla::fp8_decode_kernel(num_heads, total_tokens, cus),
      num_segments);
  if (total_tokens > 0 && workspace_bytes < plan.workspace_bytes) return FP8MLA_ERR_WORKSPACE;
  if (debug_check(kv_indptr, batch, total_tokens, kv_indices, num_slots, cus, stream) != hipSuccess)
    return FP8MLA_ERR_HIP;
  const hipError_t e = fp8mla::launch_mla_decode(q, kv_pool, num_slots, kv_indptr, kv_indices,
                                                 total_tokens, batch, num_heads, scale, sm_scale,
                                                 out, workspace, plan,
                                                 static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8MLA_OK : FP8MLA_ERR_HIP;
}

int mla_decode_fp8_noalloc(const uint16_t* q, const uint8_t* kv_pool, int64_t num_slots,
                           const int32_t* kv_indptr, const int32_t* kv_indices,
                           int64_t total_tokens, int32_t batch, int32_t num_heads, float scale,
                           float sm_scale, uint16_t* out, void* stream) {
  const int st = check_decode_fp8_args(q, kv_pool, num_slots, kv_indptr, kv_indices, total_tokens,
                                       batch, num_heads, scale, sm_scale, out);
  if (st != FP8MLA_OK) return st;
  if (batch > FP8MLA_NOALLOC_MAX_BATCH) return FP8MLA_ERR_BAD_SHAPE;
  const int cus = current_device_cus();
  if (cus <= 0) return FP8MLA_ERR_HIP;
  const fp8mla::DecodePlan plan = fp8mla::plan_mla_decode(batch, num_heads, total_tokens, cus,
                                                          fp8mla::fp8_decode_kernel(num_heads, total_tokens, cus));
  void* ws = nullptr;
  if (total_tokens > 0) {
    if (plan.workspace_bytes > kScratchBytes) return FP8MLA_ERR_WORKSPACE;
    ws = current_device_scratch();
    if (!ws) return FP8MLA_ERR_HIP;
  }
  if (debug_check(kv_indptr, batch, total_tokens, kv_indices, num_slots, cus, stream) != hipSuccess)
    return FP8MLA_ERR_HIP;
  const hipError_t e = fp8mla::launch_mla_decode(q, kv_pool, num_slots, kv_indptr, kv_indices,
                                                 total_tokens, batch, num_heads, scale, sm_scale,
                                                 out, ws, plan, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8MLA_OK : FP8MLA_ERR_HIP;
}

size_t mla_decode_bf16_workspace_bytes(int32_t batch, int32_t num_heads, int64_t total_tokens) {
  if (batch < 1 || batch > FP8MLA_MAX_BATCH || num_heads < 1 || num_heads > FP8MLA_MAX_HEADS ||
      total_tokens < 0 || total_tokens > kMaxTokens)
    return 0;
  if (total_tokens == 0) return 0;
  const int cus = current_device_cus();
  if (cus <= 0) return 0;
  return fp8mla::plan_mla_decode(batch, num_heads, total_tokens, cus, fp8mla::DecodeKernel::kBf16)
      .workspace_bytes;
}

int mla_decode_bf16(const uint16_t* q, const uint16_t* kv, int64_t num_rows,
                    const int32_t* kv_indptr, const int32_t* kv_indices, int64_t total_tokens,
                    int32_t batch, int32_t num_heads, float scale, float sm_scale, uint16_t* out,
                    void* workspace, size_t workspace_bytes, void* stream) {
  if (batch < 1 || batch > FP8MLA_MAX_BATCH || num_heads < 1 || num_heads > FP8MLA_MAX_HEADS ||
      total_tokens < 0 || total_tokens > kMaxTokens || num_rows < 0 || num_rows > kMaxSlots)
    return FP8MLA_ERR_BAD_SHAPE;
  if (total_tokens > 0 && num_rows == 0) return FP8MLA_ERR_BAD_SHAPE;
  if (!isfinite(scale) || !(scale > 0.0f) || !isfinite(sm_scale)) return FP8MLA_ERR_BAD_SCALAR;
  if (!q || !kv_indptr || !out) return FP8MLA_ERR_NULL_PTR;
  if (total_tokens > 0 && (!kv || !kv_indices || !workspace)) return FP8MLA_ERR_NULL_PTR;
  if (!aligned16(q) || !aligned16(out) || !aligned4(kv_indptr)) return FP8MLA_ERR_MISALIGNED;
  if (total_tokens > 0 && (!aligned16(kv) || !aligned4(kv_indices) || !aligned16(workspace)))
    return FP8MLA_ERR_MISALIGNED;
  const int cus = current_device_cus();
  if (cus <= 0) return FP8MLA_ERR_HIP;
  const fp8mla::DecodePlan plan =
      fp8mla::plan_mla_decode(batch, num_heads, total_tokens, cus, fp8mla::DecodeKernel::kBf16);
  if (total_tokens > 0 && workspace_bytes < plan.workspace_bytes) return FP8MLA_ERR_WORKSPACE;
  if (debug_check(kv_indptr, batch, total_tokens, kv_indices, num_rows, cus, stream) != hipSuccess)
    return FP8MLA_ERR_HIP;
  const hipError_t e = fp8mla::launch_mla_decode_bf16(q, kv, num_rows, kv_indptr, kv_indices,
                                                      total_tokens, batch, num_heads, scale,
                                                      sm_scale, out, workspace, plan,
                                                      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8MLA_OK : FP8MLA_ERR_HIP;
}

}  // extern "C"
