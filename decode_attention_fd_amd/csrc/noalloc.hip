// fd_decode_fused_noalloc: the fused decode call with its workspace and arrival
// counters in a static device array of this library instead of caller
// buffers, for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The array `scratch` below is FD_NOALLOC_SCRATCH_BYTES of device memory that
// every GPU the library runs on holds from module load until the process ends.
// Host code never uses the array's name as an address (on the host it names a
// stand-in, not device memory): the first call on each device, with that
// device current, asks hipGetSymbolAddress for that device's copy and keeps
// the pointer, and every launch takes that pointer.
//
// Layout of one call inside the array: [counters: B*Hkv uint32, 256-byte
// padded][ws_o: plan->ws_o_bytes][ws_stats: plan->ws_stats_bytes]. The
// counters are cleared by a fill kernel at the start of every call (the fused
// kernels need them zero); the workspace needs no clearing, since the fused
// kernels write every state they read. All calls on one device share the
// array, so calls that overlap in time on one device race (issue them on one
// stream).
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>

#include "fd_internal.h"

namespace fd {
namespace {

static __device__ __align__(256) unsigned char scratch[FD_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mutex;
std::map<int, void*> g_scratch_ptr;     // device -> address of its copy of `scratch`

// This device's copy of `scratch`, looked up once per device.
int scratch_for_current_device(void** out) {
  int dev = 0;
  int err = (int)hipGetDevice(&dev);
  if (err) return err;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  auto it = g_scratch_ptr.find(dev);
  if (it == g_scratch_ptr.end()) {
    void* ptr = nullptr;
    err = (int)hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (err) return err;
    if (!ptr) return (int)hipErrorInvalidSymbol;
    it = g_scratch_ptr.emplace(dev, ptr).first;
  }
  *out = it->second;
  return 0;
}

__global__ void zero_words(uint32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

constexpr int64_t kAlign = 256;
inline int64_t align_up(int64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

}  // namespace
}  // namespace fd

using namespace fd;

extern "C" FD_API int fd_decode_fused_noalloc(const fd_plan_t* plan, const fd_args* args, float* out, float* lse,
                                              void* stream) {
  int st = check_fused_plan(plan);
  if (st != FD_OK) return st;
  const int64_t ctr_bytes = align_up(plan->ws_counter_bytes);
  const int64_t o_bytes = align_up(plan->ws_o_bytes);
  const int64_t total = ctr_bytes + o_bytes + plan->ws_stats_bytes;
  if (total > (int64_t)FD_NOALLOC_SCRATCH_BYTES) return FD_ERR_WORKSPACE;
  // Every argument check of fd_decode_fused runs first, before any HIP call,
  // with a stand-in for the scratch addresses (256-byte aligned, as the real
  // ones are); the real addresses replace it afterwards.
  unsigned char* const stand_in = reinterpret_cast<unsigned char*>((uintptr_t)kAlign);
  SplitParams p;
  st = fused_params(plan, args, reinterpret_cast<float*>(stand_in), (size_t)plan->ws_o_bytes,
                    reinterpret_cast<float*>(stand_in), (size_t)plan->ws_stats_bytes,
                    reinterpret_cast<uint32_t*>(stand_in), (size_t)plan->ws_counter_bytes, out, lse, &p);
  if (st != FD_OK) return st;
  void* base = nullptr;
  int err = scratch_for_current_device(&base);
  if (err) return record_hip_error(err, "hipGetSymbolAddress(scratch)");
  unsigned char* s = static_cast<unsigned char*>(base);
  uint32_t* counters = reinterpret_cast<uint32_t*>(s);
  p.counters = counters;
  p.ws_o = reinterpret_cast<float*>(s + ctr_bytes);
  p.ws_stats = reinterpret_cast<float*>(s + ctr_bytes + o_bytes);
  const int64_t words = plan->ws_counter_bytes / 4;
  const int threads = 256;
  const int64_t blocks64 = (words + threads - 1) / threads;
  const unsigned blocks = (unsigned)(blocks64 < 1024 ? (blocks64 > 0 ? blocks64 : 1) : 1024);
  hipLaunchKernelGGL(zero_words, dim3(blocks), dim3(threads), 0, reinterpret_cast<hipStream_t>(stream), counters,
                     words);
  err = (int)hipGetLastError();
  if (err) return record_hip_error(err, "counter clear launch");
  return launch_fused(plan, p, stream);
}
