// noalloc.hip -- pct_build_tree_noalloc: the parent-conditioned build with
// its workspace in a fixed device array of this library, for callers that
// cannot allocate device memory (code under graph capture, tight serving
// loops, harnesses that forbid allocation).  Nothing here allocates.
#include <mutex>
#include <stdio.h>

#include "../../include/pctree.h"
#include "pct_internal.h"

namespace {

constexpr size_t kScratchBytes = (size_t)32 << 20;
constexpr int kMaxDevices = 64;

// One copy per GPU, alive until the process ends.  In host code this name
// is only a handle for hipGetSymbolAddress, never a device address.
__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_addr[kMaxDevices] = {};

}  // namespace

extern "C" {

pct_status pct_build_tree_noalloc(const pct_tree_shape* shape,
                                  const float* L, const void* U,
                                  const void* W, const int32_t* anchor,
                                  int32_t* tok, int32_t* parent,
                                  int32_t* depth, float* score,
                                  int32_t* n_nodes, uint64_t* mask,
                                  void* stream) {
  // host-only checks first: the shape and the size of its workspace
  const size_t need = pct_build_tree_workspace(shape);
  if (need == 0) {
    // pct_build_tree reports the reason of the invalid shape
    return pct_build_tree(shape, L, U, W, anchor, tok, parent, depth, score,
                          n_nodes, mask, nullptr, 0, stream);
  }
  if (need > kScratchBytes) {
    char msg[160];
    snprintf(msg, sizeof msg,
             "workspace of %zu bytes exceeds the fixed %zu-byte array", need,
             kScratchBytes);
    return pct::set_error(PCT_ERR_UNSUPPORTED, msg);
  }
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return pct::set_error(PCT_ERR_HIP, "no usable current device");
  }
  void* base;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_addr[dev] == nullptr) {
      // once per device, with that device current
      void* p = nullptr;
      const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || p == nullptr) {
        (void)hipGetLastError();
        char msg[160];
        snprintf(msg, sizeof msg, "hipGetSymbolAddress: %s",
                 hipGetErrorString(e));
        return pct::set_error(PCT_ERR_HIP, msg);
      }
      g_addr[dev] = p;
    }
    base = g_addr[dev];
  }
  // every kernel reads and writes the array through `base`; no part of it
  // has to start at zero (each build writes every entry before reading it)
  return pct_build_tree(shape, L, U, W, anchor, tok, parent, depth, score,
                        n_nodes, mask, base, kScratchBytes, stream);
}

}  // extern "C"
