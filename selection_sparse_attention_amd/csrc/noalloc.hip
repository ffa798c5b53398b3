// Decode entry point for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).  It runs the same kernels as sparse_attn_decode, with the
// workspace - the work items' partial (m, l, acc) rows and the per-group item
// table - carved from `scratch`, a file-scope device array of fixed size that
// each GPU holds for the life of the process.
//
// The array's name is only a host-side stand-in for it: kernels get its
// device address, looked up once per device with hipGetSymbolAddress while
// that device is current, and kept per device (each GPU has its own copy of
// the array at its own address).  Nothing here calls hipMalloc or hipFree.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "../../include/sparse_attn.h"
#include "abi_internal.hpp"

namespace {

constexpr size_t kScratchBytes = SPARSE_ATTN_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of `scratch` on each device (0: not looked up yet).  A race
// between two first calls stores the same value twice.
std::atomic<uintptr_t> g_scratch_addr[kMaxDevices];

// The current device's copy of `scratch`, or nullptr on failure.
void* scratch_on_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  uintptr_t p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p == 0) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
    p = reinterpret_cast<uintptr_t>(ptr);
    g_scratch_addr[dev].store(p, std::memory_order_release);
  }
  return reinterpret_cast<void*>(p);
}

}  // namespace

extern "C" int32_t sparse_attn_decode_noalloc(const sa_params* p, const sa_buffers* b,
                                              void* stream) {
  // size first (validates the arguments and launches nothing)
  size_t need = 0;
  int32_t st = sa::decode_entry(p, b, nullptr, &need, stream);
  if (st != SA_OK) return st;
  if (need > kScratchBytes) return SA_ERR_WORKSPACE;
  void* ws = scratch_on_current_device();
  if (!ws) return SA_ERR_HIP;
  size_t have = kScratchBytes;
  return sa::decode_entry(p, b, ws, &have, stream);
}
