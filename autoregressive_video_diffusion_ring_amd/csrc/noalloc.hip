// rc_chunk_attention_noalloc: the chunk attention with its key-split
// partials in a fixed device array instead of a caller workspace, for callers
// that cannot allocate (code under HIP graph capture, tight serving loops).
//
// The array is a file-scope __device__ object: every GPU the library runs on
// holds its own copy, at its own address, until the process ends.  Its
// address is looked up once per device (hipGetSymbolAddress, with that device
// current, on the first call there) and passed to the kernels exactly like a
// workspace.  Calls that overlap on one GPU share the array and race.  Every
// partial a call reads was written by the same call (each split writes all of
// its rows, empty splits included), so nothing needs clearing.
#include <hip/hip_runtime.h>

#include <atomic>

#include "../../include/rc.h"
#include "rc_kernels.h"

namespace {

constexpr size_t kScratchBytes = size_t(16) << 20;  // 16 MiB per GPU
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::atomic<void*> g_scratch[kMaxDevices];

template <class... A>
rc_status reject(int st, const char* fmt, A... args) {
  return static_cast<rc_status>(rc::host_fail(st, fmt, args...));
}

}  // namespace

extern "C" {

size_t rc_attention_noalloc_limit(void) { return kScratchBytes; }

rc_status rc_chunk_attention_noalloc(const rc_ring* ring, const void* q, int32_t n_q, int32_t q_pos0,
                                     int32_t q_block0, int32_t q_block_len, float cache_bias, float softmax_scale,
                                     void* out, float* lse, void* stream) {
  const size_t need = rc_attention_workspace_bytes(ring, n_q);
  if (need > kScratchBytes)
    return reject(RC_ERR_ARG, "the call needs %zu bytes of split scratch; the no-allocation entry point has %zu",
                         need, kScratchBytes);
  void* ptr = nullptr;
  if (need > 0) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return reject(RC_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return reject(RC_ERR_UNSUPPORTED, "device %d out of range", dev);
    ptr = g_scratch[dev].load(std::memory_order_acquire);
    if (!ptr) {
      e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !ptr)
        return reject(RC_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
      g_scratch[dev].store(ptr, std::memory_order_release);
    }
  }
  return rc_chunk_attention(ring, q, n_q, q_pos0, q_block0, q_block_len, cache_bias, softmax_scale, out, lse, ptr,
                            need, stream);
}

}  // extern "C"
