// kda_noalloc.hip -- kda_bwd_noalloc: the backward pass with its workspace in a static
// device array instead of a caller workspace, for callers that cannot allocate.
//
// `scratch` is a file-scope device array; each GPU the library runs on holds its own
// copy (at its own address) from the time the code object is loaded until the process
// ends.  In host code the array's name is only a host-side stand-in, so its device
// address is looked up once per device with hipGetSymbolAddress and every host use
// (here: the workspace pointer handed to kda_bwd, and through it every kernel argument)
// takes that address.  The backward's kernels write every workspace region they read
// within the same call (chunk table, per-chunk operands, partial sums), so nothing has
// to start at zero and the contents a previous call left behind are never read.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kda.h"
#include "kda_launch.h"

namespace {

__device__ __align__(256) char scratch[KDA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on first use).
int scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return KDA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return KDA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return KDA_ERR_HIP;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return KDA_OK;
}

}  // namespace

extern "C" KDA_API int kda_bwd_noalloc(const kda_problem* p, const kda_bwd_io* io, void* stream) {
  if (!io) return KDA_ERR_INVALID_ARGUMENT;
  size_t need = 0;
  int st = kda::bwd_workspace_need(p, io->h_saved != nullptr, &need);
  if (st != KDA_OK) return st;
  if (need > KDA_NOALLOC_SCRATCH_BYTES) return KDA_ERR_SCRATCH_TOO_SMALL;
  void* ws = nullptr;
  st = scratch_ptr(&ws);
  if (st != KDA_OK) return st;
  return kda_bwd(p, io, ws, KDA_NOALLOC_SCRATCH_BYTES, stream);
}
