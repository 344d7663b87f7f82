// tq_api.hip -- status strings, device cache and launch helpers of libtq.
#include <atomic>
#include <mutex>
#include <unordered_map>

#include "tq_host.h"

namespace tq {

namespace {
constexpr int kMaxDevices = 64;
std::atomic<int> g_num_cus[kMaxDevices];
std::atomic<int> g_max_shared[kMaxDevices];
}  // namespace

tq_status current_device(DeviceInfo *info) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();  // do not leave our probe's error behind
    return TQ_ERR_DEVICE;
  }
  // The CU count is published last (release), so a thread that sees it
  // (acquire) also sees the shared-memory size stored before it.
  int cus = g_num_cus[dev].load(std::memory_order_acquire);
  int shm = g_max_shared[dev].load(std::memory_order_relaxed);
  if (cus <= 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount,
                              dev) != hipSuccess ||
        cus <= 0) {
      (void)hipGetLastError();
      return TQ_ERR_DEVICE;
    }
    if (hipDeviceGetAttribute(&shm, hipDeviceAttributeMaxSharedMemoryPerBlock,
                              dev) != hipSuccess) {
      (void)hipGetLastError();
      shm = 65536;
    }
    g_max_shared[dev].store(shm, std::memory_order_relaxed);
    g_num_cus[dev].store(cus, std::memory_order_release);
  }
  info->device = dev;
  info->num_cus = cus;
  info->max_shared_per_block = shm;
  return TQ_OK;
}

tq_status allow_dynamic_lds(const void *kernel, int bytes) {
  if (bytes <= 65536) return TQ_OK;
  static std::mutex mu;
  static std::unordered_map<const void *, int> done;
  std::lock_guard<std::mutex> lock(mu);
  auto it = done.find(kernel);
  if (it != done.end() && it->second >= bytes) return TQ_OK;
  if (hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                          bytes) != hipSuccess) {
    (void)hipGetLastError();
    return TQ_ERR_LAUNCH;
  }
  done[kernel] = bytes;
  return TQ_OK;
}

}  // namespace tq

extern "C" const char *tq_status_string(tq_status s) {
  switch (s) {
    case TQ_OK: return "ok";
    case TQ_ERR_NULL: return "a required pointer is NULL";
    case TQ_ERR_SHAPE:
      return "bad shape (need N%4==0, K%16==0, 0<=K<=131072, 0<=M<=64)";
    case TQ_ERR_ALIGN:
      return "misaligned pointer (packed/xq/x need 16 B, y/acc/scales 4 B)";
    case TQ_ERR_DTYPE: return "unknown activation dtype";
    case TQ_ERR_DEVICE: return "no usable HIP device";
    case TQ_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown tq_status";
}
