// On-device validation of a request CSR (indptr) and its slot ids, for
// gfx950.  The read kernels clamp every out-of-range slot id into the pool and
// every indptr entry into its array, so a broken index layout gives wrong
// rows, never an out-of-bounds access -- and no error either.  The pages warn
// against exactly that kind of silent failure ("The KV Cache Cast
// Bottleneck", Assumptions, assumption 5: a fallback that silently does
// nothing masks configuration errors), so these kernels check the caller's
// contract on the device, without a host read of the arrays:
//   indptr[0] == 0, indptr non-decreasing, indptr[batch] == total, and
//   0 <= indices[i] < num_slots for i < total.
// Violations are recorded with device atomics in int32 status[4]:
//   [0] flags (FP8MLA_CHECK_* bits), [1] first request b with indptr[b+1] <
//   indptr[b] (INT32_MAX if none), [2] first position of an out-of-range slot
//   id (INT32_MAX if none), [3] number of out-of-range slot ids.
#include "launch.h"

#include "../../include/fp8mla.h"

namespace fp8mla {
namespace {

constexpr int CHECK_THREADS = 256;

__global__ __launch_bounds__(64) void check_reset_kernel(int32_t* __restrict__ st) {
  if (threadIdx.x < 4) st[threadIdx.x] = (threadIdx.x == 1 || threadIdx.x == 2) ? INT32_MAX : 0;
}

__global__ __launch_bounds__(CHECK_THREADS) void check_indptr_kernel(const int32_t* __restrict__ indptr,
                                                                     int32_t batch, int64_t total,
                                                                     int32_t* __restrict__ st) {
  const int64_t stride = (int64_t)gridDim.x * CHECK_THREADS;
  for (int64_t b = (int64_t)blockIdx.x * CHECK_THREADS + threadIdx.x; b <= batch; b += stride) {
    const int32_t v = indptr[b];
    int32_t f = 0;
    if (b == 0 && v != 0) f |= FP8MLA_CHECK_INDPTR_START;
    if (b == batch && (int64_t)v != total) f |= FP8MLA_CHECK_INDPTR_END;
    if (b < batch && indptr[b + 1] < v) {
      f |= FP8MLA_CHECK_INDPTR_ORDER;
      atomicMin(&st[1], (int32_t)b);
    }
    if (f) atomicOr(&st[0], f);
  }
}

__global__ __launch_bounds__(CHECK_THREADS) void check_slots_kernel(const int32_t* __restrict__ idx,
                                                                    int64_t n, uint32_t num_slots,
                                                                    int32_t* __restrict__ st) {
  const int64_t stride = (int64_t)gridDim.x * CHECK_THREADS;
  int bad = 0;
  int32_t first = INT32_MAX;
  for (int64_t i = (int64_t)blockIdx.x * CHECK_THREADS + threadIdx.x; i < n; i += stride) {
    if ((uint32_t)idx[i] >= num_slots) {  // negative ids compare as huge
      ++bad;
      first = min(first, (int32_t)i);
    }
  }
  if (bad) {
    atomicOr(&st[0], FP8MLA_CHECK_SLOT_RANGE);
    atomicMin(&st[2], first);
    atomicAdd(&st[3], bad);
  }
}

}  // namespace

hipError_t launch_index_check(const int32_t* indptr, int32_t batch, int64_t total,
                              const int32_t* indices, int64_t num_slots, int32_t* status,
                              bool reset, int num_cus, hipStream_t stream) {
  if (reset) {
    hipLaunchKernelGGL(check_reset_kernel, dim3(1), dim3(64), 0, stream, status);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (indptr) {  // (a gather's index list has no request CSR)
    const int64_t want_p = ((int64_t)batch + 1 + CHECK_THREADS - 1) / CHECK_THREADS;
    const int gp = (int)(want_p < 4 * (int64_t)num_cus ? want_p : 4 * (int64_t)num_cus);
    hipLaunchKernelGGL(check_indptr_kernel, dim3(gp), dim3(CHECK_THREADS), 0, stream, indptr, batch,
                       total, status);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!indices || total <= 0) return hipSuccess;
  // slot ids are int32: ids at or past 2^31 cannot name a slot
  const uint32_t limit =
      num_slots <= (int64_t)INT32_MAX ? (uint32_t)num_slots : (uint32_t)INT32_MAX + 1u;
  const int64_t want_s = (total + CHECK_THREADS - 1) / CHECK_THREADS;
  const int gs = (int)(want_s < 4 * (int64_t)num_cus ? want_s : 4 * (int64_t)num_cus);
  hipLaunchKernelGGL(check_slots_kernel, dim3(gs), dim3(CHECK_THREADS), 0, stream, indices, total,
                     limit, status);
  return hipGetLastError();
}

}  // namespace fp8mla
