// fa_decode_noalloc: the split-KV decode with its partial results in a device array that the
// library owns, for callers that cannot allocate device memory (code under HIP graph capture,
// serving loops, harnesses that forbid hipMalloc). The kernels are fa_decode's.
#include <mutex>

#include "fa.h"
#include "fa_launch.h"

namespace {

constexpr size_t kScratchBytes = FA_DECODE_NOALLOC_SCRATCH_BYTES;

// Per-split partial outputs and log-sum-exps ([B, H, splits, d] then [B, H, splits] fp32, the
// layout of fa_decode's workspace). Every GPU the library runs on holds its own copy until the
// process ends. In host code this name is not a device address: the address of each device's copy
// comes from hipGetSymbolAddress (scratch_address below), and only that is ever passed on.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void* g_scratch[kMaxDevices] = {};  // device address of each device's copy, once looked up

// The address of `scratch` on the device that runs `stream`, looked up once per device with that
// device current (the caller's current device is restored).
hipError_t scratch_address(hipStream_t stream, void** out) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  int dev = cur;
  if (stream != nullptr) {
    e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return e;
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> guard(g_lock);
  if (g_scratch[dev] == nullptr) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

extern "C" fa_status fa_decode_noalloc(const fa_bf16* q, const fa_bf16* k, const fa_bf16* v,
                                       fa_bf16* o, float* lse, int B, int H, int N_q, int N_k,
                                       int d, float scale, int causal, int num_splits,
                                       hipStream_t stream) {
  int c = 0;
  const fa_status s =
      fa::decode_validate(q, k, v, o, lse, B, H, N_q, N_k, d, scale, causal, num_splits, &c);
  if (s != FA_OK) return s;
  if (fa_decode_workspace_bytes(B, H, N_k, d, c) > kScratchBytes) return FA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (scratch_address(stream, &ws) != hipSuccess) return FA_ERR_HIP;
  // the split kernel writes every partial it owns (an empty split writes o = 0, L = -inf) before
  // the combine reads it, so the array needs no clearing between calls
  return fa::decode_run(q, k, v, o, lse, ws, B, H, N_k, d, scale, c, stream);
}
