// Static device scratch of the allocation-free pick-rule entry point (he_sample_static).
//
// Some callers cannot allocate device memory (work under graph capture, tight serving
// loops, harnesses that forbid it).  For them the pick rule on caller logits runs on a
// file-scope device array instead of the workspace.  Each GPU the library runs on
// holds its own copy until the process ends; its address on a device is taken once,
// with that device current, by hipGetSymbolAddress, and only that address is handed to
// kernels (the array's name is a host-side stand-in in host code).
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace he {

namespace {

// layout: the position pair (256 bytes), then five [kStaticRows * kStaticBlocks] arrays
constexpr size_t kPart = (size_t)kStaticRows * kStaticBlocks * 4;
constexpr size_t kStaticBytes = 256 + 5 * kPart;

__device__ __align__(256) char scratch[kStaticBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
char* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t static_scratch(int device, StaticScratch* out) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[device]) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != device && (e = hipSetDevice(device)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != device) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[device] = static_cast<char*>(p);
  }
  char* b = g_ptr[device];
  out->pos = reinterpret_cast<int32_t*>(b);
  out->best_val = reinterpret_cast<float*>(b + 256);
  out->best_idx = reinterpret_cast<int32_t*>(b + 256 + kPart);
  out->best_lg = reinterpret_cast<float*>(b + 256 + 2 * kPart);
  out->blk_max = reinterpret_cast<float*>(b + 256 + 3 * kPart);
  out->blk_sum = reinterpret_cast<float*>(b + 256 + 4 * kPart);
  return hipSuccess;
}

size_t static_scratch_bytes() { return kStaticBytes; }

}  // namespace he
