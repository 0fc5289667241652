// Allocation-free variant of the active-query attention entry point, for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid allocation).  The kernels are
// those of hsa_attn_active; the KV-split partials it would keep in a caller
// workspace live instead in `scratch`, a file-scope device array of fixed
// size that each GPU holds from the library's load until the process ends.
//
// The array's name is only a host-side handle: its device address is looked
// up once per device (hipGetSymbolAddress, with that device current) and that
// address is what the kernels receive.  Every call on one GPU shares its
// array, so calls that overlap on one GPU (two streams, two threads) race on
// it; nothing in it has to start at zero (each partial the merge reads is
// written by the same call first).
#include <math.h>

#include <mutex>

#include "common.h"

using namespace hsa;

namespace {

constexpr size_t kScratchBytes = HSA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch`, per device

// Device address of `scratch` on the current device (looked up on first use).
hsa_status current_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return HSA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return HSA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return HSA_OK;
}

}  // namespace

extern "C" hsa_status hsa_attn_active_noalloc(const void* q, const void* k, const void* v, void* o,
                                              int32_t n_active, int32_t n_kv, int32_t H,
                                              int32_t Dh, float scale, hsa_dtype dtype,
                                              void* stream) {
  if (dtype != HSA_F32 && dtype != HSA_BF16) return HSA_ERR_DTYPE;
  if (n_active < 0 || n_kv <= 0 || H <= 0 || (Dh != 64 && Dh != 128)) return HSA_ERR_SHAPE;
  if (dtype == HSA_BF16 && (int64_t)n_kv * H * Dh * 2 >= ((int64_t)1 << 32)) return HSA_ERR_SHAPE;
  if (n_active == 0) return HSA_OK;
  for (const void* p : {q, k, v, (const void*)o}) {
    if (p == nullptr) return HSA_ERR_ARG;
    if (!aligned16(p)) return HSA_ERR_ALIGN;
  }
  if (!(scale > 0.f) || !isfinite(scale)) return HSA_ERR_ARG;
  const size_t need = dtype == HSA_BF16 ? attn_workspace_bytes(n_active, n_kv, H, Dh) : 0;
  if (need > kScratchBytes) return HSA_ERR_TOO_LARGE;
  void* ws = nullptr;
  if (need > 0) {
    const hsa_status st = current_scratch(&ws);
    if (st != HSA_OK) return st;
  }
  return launch_attention(q, k, v, o, n_active, n_kv, H, Dh, scale, dtype, ws, kScratchBytes,
                          reinterpret_cast<hipStream_t>(stream));
}
