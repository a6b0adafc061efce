// wq_gemm_noalloc: the dense product for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  The
// scratch wq_gemm takes from the caller (the act_order gather buffer and the split-K fp32
// partials) comes instead from one file-scope device array, `scratch`, of kScratchBytes on
// each GPU, held until the process ends.  Every call on a GPU shares that GPU's array, so
// calls that overlap on one GPU race; its contents are never assumed (neither use needs
// zeroed memory).
#include <hip/hip_runtime.h>

#include <mutex>

#include "wq.h"
#include "wq_internal.h"

namespace {

constexpr size_t kScratchBytes = WQ_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of `scratch` on each device (the host-side name is only a stand-in): taken
// once per device, with that device current, by hipGetSymbolAddress.
void* g_scratch[kMaxDevices] = {};
std::mutex g_scratch_mutex;

int scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return WQ_STATUS(WQ_STAGE_DEVICE, (int)e);
  if (dev < 0 || dev >= kMaxDevices) return WQ_STATUS(WQ_STAGE_DEVICE, (int)hipErrorInvalidDevice);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return WQ_STATUS(WQ_STAGE_DEVICE, (int)e);
    if (ptr == nullptr) return WQ_STATUS(WQ_STAGE_DEVICE, (int)hipErrorInvalidSymbol);
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return 0;
}

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

extern "C" {

int wq_gemm_noalloc(const wq_gemm_args* args) {
  if (args == nullptr) return WQ_STATUS(WQ_STAGE_ARGS, WQ_ERR_NULL);
  if (args->abi_version != WQ_ABI_VERSION || args->struct_size != sizeof(wq_gemm_args) ||
      args->reserved != 0)
    return WQ_STATUS(WQ_STAGE_ARGS, WQ_ERR_ABI);
  // the scratch comes from the library: the caller's scratch fields must be empty
  if (args->workspace != nullptr || args->workspace_bytes != 0 || args->a_tmp != nullptr)
    return WQ_STATUS(WQ_STAGE_ARGS, WQ_ERR_WORKSPACE);
  int32_t kernel = 0, splits = 0;
  int st = wq_gemm_plan(args->m, args->n, args->k, args->group_size, args->flags,
                        args->split_k, &kernel, &splits);
  if (st) return st;
  const bool act_order = (args->flags & WQ_FLAG_ACT_ORDER) != 0;
  const size_t gather = act_order ? round256((size_t)args->m * args->k * 2) : 0;
  if (gather > kScratchBytes) return WQ_STATUS(WQ_STAGE_ARGS, WQ_ERR_WORKSPACE);
  const size_t per_split = (size_t)args->m * args->n * sizeof(float);
  int32_t split_k = args->split_k;
  if (splits > 1 && (size_t)splits * per_split > kScratchBytes - gather && split_k == 0) {
    // the library's own split does not fit: the largest split that does (or none)
    const size_t fit = (kScratchBytes - gather) / per_split;
    split_k = fit >= 2 ? (int32_t)(fit < (size_t)splits ? fit : (size_t)splits) : 1;
    if ((st = wq_gemm_plan(args->m, args->n, args->k, args->group_size, args->flags, split_k,
                           &kernel, &splits)))
      return st;
  }
  const size_t partials = splits > 1 ? (size_t)splits * per_split : 0;
  if (partials > kScratchBytes - gather) return WQ_STATUS(WQ_STAGE_ARGS, WQ_ERR_WORKSPACE);
  void* base = nullptr;
  if ((st = scratch_for_current_device(&base))) return st;
  wq_gemm_args p = *args;
  p.split_k = split_k;
  unsigned char* bytes = static_cast<unsigned char*>(base);
  p.a_tmp = act_order ? bytes : nullptr;
  p.workspace = partials ? bytes + gather : nullptr;
  p.workspace_bytes = partials ? kScratchBytes - gather : 0;
  return wq_gemm(&p);
}

}  // extern "C"
