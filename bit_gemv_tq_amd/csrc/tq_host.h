// tq_host.h -- host-side helpers of libtq: argument checks, the per-device
// compute-unit cache and a launch wrapper that reports launch failures.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "../../include/tq.h"

namespace tq {

inline bool aligned(const void *p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

// Shape rules common to every weight-consuming call.
inline tq_status check_nk(int64_t N, int64_t K) {
  if (N < 0 || K < 0) return TQ_ERR_SHAPE;
  if (N % 4 != 0) return TQ_ERR_SHAPE;
  if (K % 16 != 0) return TQ_ERR_SHAPE;
  if (K > TQ_MAX_K) return TQ_ERR_SHAPE;
  if (N / 4 > (int64_t)INT32_MAX) return TQ_ERR_SHAPE;
  return TQ_OK;
}

inline tq_status check_m(int64_t M) {
  return (M < 0 || M > TQ_MAX_M) ? TQ_ERR_SHAPE : TQ_OK;
}

struct DeviceInfo {
  int device = -1;
  int num_cus = 0;
  int max_shared_per_block = 0;
};

// Current device and its CU count (queried once per device, then cached).
tq_status current_device(DeviceInfo *info);

// Launch `kernel` with `args...`; maps a launch failure to TQ_ERR_LAUNCH.
template <typename... Params, typename... Args>
tq_status launch(void (*kernel)(Params...), dim3 grid, dim3 block,
                 size_t shmem, hipStream_t stream, Args... args) {
  static_assert(sizeof...(Params) == sizeof...(Args), "argument count");
  // Convert every argument to the kernel's parameter type, then hand HIP an
  // array of pointers to those values.
  auto call = [&](Params... p) -> tq_status {
    void *ptrs[] = {static_cast<void *>(&p)..., nullptr};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(kernel),
                                   grid, block, ptrs, shmem, stream);
    return e == hipSuccess ? TQ_OK : TQ_ERR_LAUNCH;
  };
  return call(static_cast<Params>(args)...);
}

// Blocks of `kernel` (launched with `threads` threads, no dynamic LDS) that
// one CU holds, asked of the runtime once and kept in `cache` (0: not asked
// yet, -1: unknown).  Persistent grids are capped at this times the CU
// count, so that no block of them waits for a second wave.
template <typename K>
int resident_blocks(K kernel, int threads, std::atomic<int> &cache) {
  int n = cache.load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, 0) != hipSuccess ||
        n < 1) {
      (void)hipGetLastError();
      n = -1;
    }
    cache.store(n, std::memory_order_relaxed);
  }
  return n;
}

// RMSNorm-folded quantization of M rows (tq_act_quant.hip), used by the
// fused GEMV's fallback; check_rms validates gamma, eps and K for both.
tq_status rmsnorm_act_quant(const void *x, tq_dtype xt, const void *gamma, float eps,
                            int64_t M, int64_t K, int8_t *xq, float *x_scale,
                            hipStream_t stream);
tq_status check_rms(const void *gamma, float eps, int64_t K);

// Allow dynamic LDS above the default limit for `kernel` (once per process
// and kernel; harmless when the request is below the default).
tq_status allow_dynamic_lds(const void *kernel, int bytes);

}  // namespace tq
