// Device-side error flags.  The kernels skip bad device data as they always
// did (a table entry inside a context that is -1 or outside the pool, a row
// whose table slot is out of range, a device context length beyond the
// table: masked, never an out-of-bounds access) and now also set a bit in
// one word that the library owns on each device; pkv_device_errors reads and
// clears it.  Source: "The path of one inference", step (4) (a block table
// holds -1 for unassigned entries, which a context must not contain).
#include <atomic>
#include <mutex>

#include "common.h"

namespace pkv {
namespace {

// One 256-byte line per device; word 0 holds the flags.  In host code the
// name is a stand-in for the symbol, not a device address: kernels receive
// the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint32_t device_error_flags[64];

constexpr int kMaxDevices = 64;
std::atomic<uint32_t*> g_flags[kMaxDevices];
std::mutex g_flags_mu;

__global__ void clear_flags_kernel(uint32_t* f) {
  if (threadIdx.x == 0) f[0] = 0;
}

}  // namespace

uint32_t* device_errors_ptr() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  uint32_t* p = g_flags[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_flags_mu);
  p = g_flags[dev].load(std::memory_order_relaxed);
  if (!p) {
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(device_error_flags)) != hipSuccess) return nullptr;
    p = static_cast<uint32_t*>(q);
    g_flags[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace pkv

using namespace pkv;

extern "C" int pkv_device_errors(uint32_t* flags_host, int clear, void* stream) {
  if (!flags_host) return PKV_ERR_NULL;
  uint32_t* p = device_errors_ptr();
  if (!p) return PKV_ERR_HIP;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(flags_host, p, sizeof(uint32_t), hipMemcpyDeviceToHost, st) != hipSuccess) return PKV_ERR_HIP;
  if (clear) {
    void* args[] = {&p};
    const int rc = launch_status(hipLaunchKernel((const void*)clear_flags_kernel, dim3(1), dim3(64), args, 0, st));
    if (rc != PKV_OK) return rc;
  }
  return hipStreamSynchronize(st) == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}
