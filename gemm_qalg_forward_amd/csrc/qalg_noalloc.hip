// qalg_forward_noalloc: the forward projection for callers that cannot
// allocate device memory (code under HIP graph capture, serving loops,
// harnesses that forbid hipMalloc).  The only scratch memory the forward needs
// is the type index it builds from tau; here that index lives in a
// library-owned device array instead of a caller workspace.
//
// The array is a file-scope __device__ variable: each GPU the library runs on
// holds its own copy (reserved with the code object, kept until the process
// ends).  Host code never passes the variable's name to a kernel (on the host
// that name is only a stand-in, not a device address): the first call on a
// device, with that device current, asks the runtime for the array's address
// on that device (hipGetSymbolAddress) and keeps it; every launch then takes
// that address as its workspace pointer.
#include <mutex>

#include "qalg.h"
#include "qalg_internal.h"

namespace {

constexpr size_t kScratchBytes = QALG_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// Address of this device's copy of `scratch` (looked up once per device, with
// the device current); nullptr if the lookup fails.
void* scratch_on(int dev) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] != nullptr) return g_ptr[dev];
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return nullptr;
  if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
  void* p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (cur != dev) (void)hipSetDevice(cur);
  if (e != hipSuccess || p == nullptr) return nullptr;
  g_ptr[dev] = p;
  return p;
}

}  // namespace

extern "C" qalg_status qalg_forward_noalloc(const void* X, const void* W, const int32_t* tau, int32_t q, int64_t M,
                                            int64_t K, int64_t N, void* Y, int32_t dtype, uint32_t flags,
                                            void* stream) {
  // another call may have replaced the index since: it is always rebuilt
  if (flags & QALG_FLAG_INDEX_READY) return QALG_ERR_ARG;
  // every argument check of qalg_forward, with no workspace: that call returns
  // an argument error, QALG_OK for M = 0 (nothing to do), or, with valid
  // arguments, QALG_ERR_NULL for the missing workspace, all before any launch
  const qalg_status dry = qalg_forward(X, W, tau, q, M, K, N, Y, dtype, nullptr, 0, flags, stream);
  if (dry != QALG_ERR_NULL) return dry;
  if (X == nullptr || W == nullptr || tau == nullptr || Y == nullptr) return QALG_ERR_NULL;
  if (qalg_workspace_bytes(q, M) > kScratchBytes) return QALG_ERR_WORKSPACE;
  // the stream's device (the current one for the null stream)
  int dev = -1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (s != nullptr) {
    hipDevice_t d;
    if (hipStreamGetDevice(s, &d) != hipSuccess) return QALG_ERR_HIP;
    dev = int(d);
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return QALG_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return QALG_ERR_HIP;
  void* ws = scratch_on(dev);
  if (ws == nullptr) return QALG_ERR_HIP;
  return qalg_forward(X, W, tau, q, M, K, N, Y, dtype, ws, kScratchBytes, flags, stream);
}
