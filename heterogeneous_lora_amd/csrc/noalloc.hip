// slora_apply_noalloc: slora_apply for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc). Its kernels are slora_apply's; the workspace they use (the decode
// launch's tagged v words, the prefill launches' k-range partial sums, the give-up
// header) is `scratch`, a static device array of kScratchBytes that every GPU the
// library runs on holds until the process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory: its device
// address is resolved once per device with hipGetSymbolAddress, with that device
// current, and only that address is ever handed to kernels or copies.
#include <map>
#include <mutex>

#include "guard.h"
#include "internal.h"

namespace slora {
namespace {

constexpr int64_t kScratchBytes = int64_t(64) << 20;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_mu;
std::map<int, void*> g_ptr;  // per device: the device address of scratch

int current_device(int* dev) {
  const hipError_t e = hipGetDevice(dev);
  return e == hipSuccess ? SLORA_OK : hip_fail(e, "hipGetDevice");
}

// Set-up on a device's first allocation-free call: resolve scratch's address with that
// device current and clear the array (the decode hand-off needs every word of it to
// start without a call's tag), on the caller's stream.
int resolve(hipStream_t s, void** out) {
  int dev = 0;
  int rc = current_device(&dev);
  if (rc) return rc;
  std::lock_guard<std::mutex> lk(g_mu);
  auto it = g_ptr.find(dev);
  if (it != g_ptr.end()) {
    *out = it->second;
    return SLORA_OK;
  }
  void* p = nullptr;
  hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
  if (!p) return fail(SLORA_E_HIP, "hipGetSymbolAddress(scratch) returned NULL");
  e = launch_zero(p, kScratchBytes, s);
  if (e != hipSuccess) return hip_fail(e, "scratch clear");
  g_ptr[dev] = p;
  *out = p;
  return SLORA_OK;
}

}  // namespace

int shared_scratch(void** ptr, int64_t* bytes) {
  if (bytes) *bytes = kScratchBytes;
  int dev = 0;
  const int rc = current_device(&dev);
  if (rc) return rc;
  std::lock_guard<std::mutex> lk(g_mu);
  auto it = g_ptr.find(dev);
  *ptr = it == g_ptr.end() ? nullptr : it->second;
  return SLORA_OK;
}

}  // namespace slora

extern "C" int slora_apply_noalloc(const slora_lora* lora, const slora_routing* routing,
                                   const void* x, void* y, void* stream) {
  return slora::guarded(__func__, [&] {
    slora::clear_error();
    if (!lora || !routing) return slora::fail(SLORA_E_INVALID, "apply_noalloc: lora / routing is NULL");
    const int64_t need = slora::ws_layout(lora, routing).total;
    if (need > slora::kScratchBytes)
      return slora::fail(SLORA_E_INVALID,
                         "apply_noalloc: the call needs %lld bytes of workspace, more than the "
                         "%lld-byte static scratch (fewer tokens per call, or slora_apply with a "
                         "caller-owned workspace)",
                         (long long)need, (long long)slora::kScratchBytes);
    void* ws = nullptr;
    const int rc = slora::resolve((hipStream_t)stream, &ws);
    if (rc) return rc;
    return slora::apply_shared(lora, routing, x, y, ws, slora::kScratchBytes, stream);
  });
}
