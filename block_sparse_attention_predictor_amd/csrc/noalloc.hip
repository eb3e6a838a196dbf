// Selection for callers that cannot allocate device memory: veda_select with its
// workspace (the projected pooled vectors q_hat and k_hat) in a fixed array that the
// library owns, instead of a caller-supplied buffer.
//
// The array is a file-scope __device__ variable: every GPU the library runs on holds
// its own copy from the time the library's code is loaded on it until the process ends.
// Host code never passes the array's name to a kernel (on the host that name is only a
// stand-in, not a device address): the device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and kept.
#include "../../include/veda.h"

#include <hip/hip_runtime.h>

#include <mutex>

namespace {

static_assert(VEDA_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size must keep 256-byte alignment");
__device__ __align__(256) unsigned char scratch[VEDA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};   // device address of `scratch` per device, 0 until looked up

// Device address of the current device's copy of `scratch`.
int scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return VEDA_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return VEDA_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return VEDA_EHIP;
    if ((reinterpret_cast<uintptr_t>(p) & 255u) != 0) return VEDA_EHIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return VEDA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" int veda_select_noalloc(const veda_layer* layer, const void* q, const void* k, const void* wq,
                                   const void* wk, int32_t* idx, float* scores_opt, void* stream) {
  // every check veda_select makes, and the size limit, before any device call
  int st = veda_layer_check(layer, 1);
  if (st != VEDA_OK) return st;
  if (!q || !k || !wq || !wk || !idx) return VEDA_EINVAL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(wq) || !aligned16(wk) || !aligned16(idx))
    return VEDA_EINVAL;
  if (scores_opt && !aligned16(scores_opt)) return VEDA_EINVAL;
  if (veda_select_workspace_bytes(layer) > (size_t)VEDA_NOALLOC_SCRATCH_BYTES) return VEDA_EWORKSPACE;
  void* ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st != VEDA_OK) return st;
  // pool/project writes every q_hat and k_hat entry before the scoring kernel reads it,
  // so nothing left in the array by an earlier call is ever read
  return veda_select(layer, q, k, wq, wk, idx, scores_opt, ws, (size_t)VEDA_NOALLOC_SCRATCH_BYTES, stream);
}
