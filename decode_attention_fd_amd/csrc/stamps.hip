// The measurement build's per-workgroup stamp records (stamps.h) and
// fd_wg_stamps, which copies them out. In the release build fd_wg_stamps
// returns FD_ERR_UNSUPPORTED and no launch records anything.
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>

#include "fd_internal.h"

namespace fd {

#ifdef FD_WG_STAMPS
namespace {

static __device__ __align__(256) uint64_t wg_stamp_records[FD_WG_STAMP_RECORDS * 4];

std::mutex g_mutex;
std::map<int, uint64_t*> g_ptr;     // device -> its copy of wg_stamp_records

uint64_t* records_for_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lock(g_mutex);
  auto it = g_ptr.find(dev);
  if (it == g_ptr.end()) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(wg_stamp_records)) != hipSuccess) ptr = nullptr;
    it = g_ptr.emplace(dev, static_cast<uint64_t*>(ptr)).first;
  }
  return it->second;
}

}  // namespace

uint64_t* wg_stamp_records_for(int64_t workgroups) {
  return workgroups <= FD_WG_STAMP_RECORDS ? records_for_current_device() : nullptr;
}

#else

uint64_t* wg_stamp_records_for(int64_t) { return nullptr; }

#endif

}  // namespace fd

extern "C" FD_API int fd_wg_stamps(void* dst, size_t dst_bytes, void* stream) {
#ifdef FD_WG_STAMPS
  if (!dst) return FD_ERR_INVALID_ARG;
  uint64_t* src = fd::wg_stamp_records_for(0);
  if (!src) return fd::record_hip_error((int)hipErrorInvalidSymbol, "hipGetSymbolAddress(wg_stamp_records)");
  size_t n = (size_t)FD_WG_STAMP_RECORDS * 32;
  if (dst_bytes < n) n = dst_bytes;
  const int err = (int)hipMemcpyAsync(dst, src, n, hipMemcpyDeviceToDevice, static_cast<hipStream_t>(stream));
  if (err) return fd::record_hip_error(err, "hipMemcpyAsync(wg stamps)");
  return FD_OK;
#else
  (void)dst;
  (void)dst_bytes;
  (void)stream;
  return FD_ERR_UNSUPPORTED;
#endif
}
