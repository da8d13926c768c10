// Entry points that allocate nothing, for callers that cannot allocate
// device memory (code under HIP graph capture, tight training loops,
// harnesses that forbid hipMalloc).  Their kernels take scratch memory from a
// fixed, file-scope device array instead of a caller-owned workspace.
//
// The array exists once per GPU the library runs on and lives until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it is only a stand-in for the symbol): the device address is looked up
// once per device with hipGetSymbolAddress, with that device current, and
// kept; kernels and copies get that address.  Every call on one GPU shares
// that GPU's array, so calls that overlap in time on one GPU (on different
// streams, or from different threads) race on it; calls ordered on one
// stream do not.
#include <mutex>

#include "common.h"

namespace {

constexpr size_t kScratchBytes = (size_t)48 << 20;  // 48 MiB per GPU
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of this GPU's scratch array (looked up on the first call on
// each device).
mt_status scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MT_E_HIP;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MT_E_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MT_OK;
}

}  // namespace

extern "C" size_t mtk_noalloc_scratch_bytes(void) { return kScratchBytes; }

extern "C" mt_status mtk_rmsnorm_bwd_noalloc(const float* dn, const float* x, const float* rstd,
                                             const uint16_t* g, const float* resid, float* dx,
                                             uint16_t* dx_bf16, float* dg, int64_t T, int32_t h,
                                             void* stream) {
  if (!dn || !x || !rstd || !g || !dx || !dg || T < 1 || h < 4 || h % 4 || h > 16384)
    return MT_E_ARG;
  // the per-workgroup column partials must fit the fixed scratch
  if (mt::rmsnorm_bwd_partial_bytes(T, h) > kScratchBytes) return MT_E_NOMEM;
  void* ws = nullptr;
  const mt_status r = scratch_ptr(&ws);
  if (r != MT_OK) return r;
  // every partial the column sums read is written first by the row kernel of
  // the same call, so nothing needs clearing between calls
  return mt::launch_rmsnorm_bwd(dn, x, rstd, g, resid, dx, dx_bf16, dg, nullptr,
                                static_cast<float*>(ws), T, h, (hipStream_t)stream) == hipSuccess
             ? MT_OK
             : MT_E_HIP;
}
