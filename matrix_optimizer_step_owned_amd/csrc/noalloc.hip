// Allocation-free gradient clipping: dmuon_clip_grad_norm_noalloc.
//
// The same computation as dmuon_clip_grad_norm (the Training Guide's global
// p-norm clip per bucket), for callers that cannot allocate: the clip's
// scratch -- the gradient table, the per-bucket block ranges and max_norm
// values, one fp64 partial per 64 KB block and the per-bucket coefficients --
// lives in `scratch`, a device array the library holds on every GPU it runs
// on, and the launch table reaches it as kernel arguments (no pinned staging
// buffer, no copy from host memory).
#include <cstring>
#include <map>
#include <mutex>
#include <vector>

#include "../../include/dmuon.h"
#include "internal.h"

namespace dmuon {
namespace {

static_assert(DMUON_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");

// Device-side scratch, one copy per GPU, kept until the process ends.  Host
// code never uses this name as an address: it uses the pointer that
// hipGetSymbolAddress returned for the current device.
static __device__ __align__(256) char scratch[DMUON_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
std::map<int, void*> g_scratch_ptr;   // device -> address of that device's scratch

// The current device's scratch address (looked up once per device).
int scratch_for_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_last_error(DMUON_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it != g_scratch_ptr.end()) {
    *out = it->second;
    return DMUON_OK;
  }
  void* ptr = nullptr;
  e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || ptr == nullptr)
    return set_last_error(DMUON_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") +
                                             (e != hipSuccess ? hipGetErrorString(e) : "null address"));
  g_scratch_ptr.emplace(dev, ptr);
  *out = ptr;
  return DMUON_OK;
}

// One piece of a launch table, passed by value: the kernel copies it from
// its argument segment to device memory.
struct ArgChunk {
  uint4 v[kArgChunkBytes / 16];
};

__global__ void __launch_bounds__(kArgChunkBytes / 16)
table_write_kernel(ArgChunk c, uint4* __restrict__ dst, int n16) {
  const int i = threadIdx.x;
  if (i < n16) dst[i] = c.v[i];
}

}  // namespace

hipError_t upload_by_kernel_args(void* dst, const void* host, size_t bytes, hipStream_t stream) {
  if (bytes % 16 || reinterpret_cast<uintptr_t>(dst) % 16) return hipErrorInvalidValue;
  const char* src = static_cast<const char*>(host);
  for (size_t off = 0; off < bytes; off += kArgChunkBytes) {
    const size_t len = std::min<size_t>(kArgChunkBytes, bytes - off);
    ArgChunk c;
    std::memset(&c, 0, sizeof c);
    std::memcpy(&c, src + off, len);
    hipLaunchKernelGGL(table_write_kernel, dim3(1), dim3(kArgChunkBytes / 16), 0, stream, c,
                       reinterpret_cast<uint4*>(static_cast<char*>(dst) + off), static_cast<int>(len / 16));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace dmuon

using namespace dmuon;

extern "C" int dmuon_clip_grad_norm_noalloc(const dmuon_grad_t* grads, int32_t n, int32_t nbuckets,
                                            const double* max_norm, double norm_type, double* total_norm,
                                            void* stream) {
  return clip_grad_norm_in_scratch(grads, n, nbuckets, max_norm, norm_type, total_norm, scratch_for_current_device,
                                   DMUON_NOALLOC_SCRATCH_BYTES, stream);
}
