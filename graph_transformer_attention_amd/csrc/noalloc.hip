// The backward with its scratch memory in a fixed device array instead of a caller's
// workspace (gt_attn_bwd_static), for callers that cannot allocate device memory:
// code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
//
// The array is a file-scope __device__ variable, so each GPU the library runs on holds
// its own copy (kScratchBytes) from the first call on that GPU until the process ends.
// In host code the array's name is only a stand-in for that symbol, not a device
// address: the first call on each device looks the address up with hipGetSymbolAddress
// (that device current) and every later call uses the address kept for the device.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "../../include/gt_attn.h"
#include "gt_internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(128) << 20;  // GT_BWD_STATIC_SCRATCH_BYTES
static_assert(kScratchBytes == GT_BWD_STATIC_SCRATCH_BYTES, "header and library disagree on the scratch size");
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of this device's scratch array, looked up once per device.
hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

extern "C" int gt_attn_bwd_static(const void* q, const void* k, const void* v, const uint8_t* spd,
                                  const uint8_t* spd_t, const float* table, const float* out, const float* lse,
                                  const void* dout, float* dq, float* dk, float* dv, float* dtable, int64_t N,
                                  int32_t H, int32_t D, int32_t NB, int32_t dtype, void* stream) {
  const size_t need = gt_attn_bwd_workspace_bytes(N, H, D, NB, dtype);
  if (need == 0) {  // invalid sizes: let the workspace entry point name the argument
    return gt_attn_bwd(q, k, v, spd, spd_t, table, out, lse, dout, dq, dk, dv, dtable, nullptr, 0, N, H, D, NB,
                       dtype, stream);
  }
  // gt_attn_bwd's own layout when it fits (same kernels, same bits); else the three-pass
  // layout, which has no room for the one-pass backward's dQ partials
  const bool fused_fits = need <= kScratchBytes;
  const size_t need3 = gt::bwd_workspace(N, N, H, D, NB, dtype, false).bytes;
  if (!fused_fits && need3 > kScratchBytes) {
    char buf[256];
    snprintf(buf, sizeof buf,
             "gt_attn_bwd_static: N=%lld, H=%d, D=%d, NB=%d needs %zu bytes of scratch, more than the fixed "
             "%zu; use gt_attn_bwd with a workspace",
             (long long)N, H, D, NB, need3, kScratchBytes);
    gt::set_last_error(buf);
    return GT_EINVAL;
  }
  void* ws = nullptr;
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) {
    char buf[256];
    snprintf(buf, sizeof buf, "gt_attn_bwd_static: scratch address lookup failed: %s", hipGetErrorString(e));
    gt::set_last_error(buf);
    return GT_EHIP;
  }
  return gt::bwd_call(q, k, v, spd, spd_t, table, out, lse, dout, dq, dk, dv, dtable, ws, kScratchBytes, N, H, D, NB,
                      dtype, stream, fused_fits);
}
