// moe_forward_noalloc: moe_forward_ex for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc). Its workspace is `scratch`, a static
// device array of MOE_NOALLOC_SCRATCH_BYTES that every GPU the library runs
// on holds until the process ends. The forward's kernels are the ones
// moe_forward_ex launches; they take the array's device address as their
// workspace pointer.
//
// The name `scratch` is a host-side stand-in in host code, not a device
// address: the address is taken once per device with hipGetSymbolAddress
// (with that device current) and only that address is ever passed on.
#include <mutex>

#include "../../include/moe_topk_ids.h"
#include "moe_internal.h"

namespace {

constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of this device's copy of `scratch`.
int scratch_for_current_device(void** out) {
  int dev = 0;
  hipError_t st = hipGetDevice(&dev);
  if (st != hipSuccess)
    return moe::set_last_error(MOE_ERR_HIP, "moe_forward_noalloc: hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices)
    return moe::set_last_error(MOE_ERR_UNSUPPORTED, "moe_forward_noalloc: device index too large");
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    st = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (st != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return moe::set_last_error(MOE_ERR_HIP,
                                 "moe_forward_noalloc: hipGetSymbolAddress of the static scratch "
                                 "array failed");
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" int moe_forward_noalloc(const void* hidden, const void* w1, const void* w2,
                                   const float* topk_weights, const int32_t* topk_ids,
                                   int64_t T, int64_t H, int64_t I, int64_t E, int64_t K,
                                   float* out, uint32_t flags, void* stream) {
  flags &= ~MOE_FLAG_FP8_WEIGHTS;  // bf16 weights, as moe_forward_ex
  const size_t need = moe_workspace_bytes(T, H, I, E, K, flags);
  if (need == 0) {
    // invalid sizes (the error is already set) or T == 0 (a no-op)
    return moe_forward_ex(hidden, w1, w2, topk_weights, topk_ids, T, H, I, E, K, out, flags,
                          nullptr, 0, stream);
  }
  if (need > kScratchBytes) {
    char msg[256];
    snprintf(msg, sizeof(msg),
             "moe_forward_noalloc: T=%lld H=%lld I=%lld E=%lld K=%lld needs %zu bytes of "
             "workspace; the static scratch holds %zu (use moe_forward_ex with a caller "
             "workspace)",
             (long long)T, (long long)H, (long long)I, (long long)E, (long long)K, need,
             kScratchBytes);
    return moe::set_last_error(MOE_ERR_WORKSPACE, msg);
  }
  void* ws = nullptr;
  const int rc = scratch_for_current_device(&ws);
  if (rc != MOE_OK) return rc;
  return moe_forward_ex(hidden, w1, w2, topk_weights, topk_ids, T, H, I, E, K, out, flags, ws,
                        kScratchBytes, stream);
}
