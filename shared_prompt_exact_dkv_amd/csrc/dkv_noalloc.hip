// dkv_noalloc.hip -- dkv_bwd_noalloc: the Call-2 backward without a caller workspace and
// without any allocation, for callers that cannot allocate (code that must not call
// hipMalloc, serving loops, harnesses that forbid allocation).
//
// The scratch space dkv_bwd takes from its workspace (the rows' -D and -LSE / scale
// terms, the work lists and tables, the split mode's slices) lives here in one
// file-scope device array of kScratchBytes.  Host code never passes the array's name
// to a kernel (on the host it names a stand-in, not device memory): the array's device
// address is looked up once per device with hipGetSymbolAddress and kept.  The work
// lists are copied from pageable host memory, a copy HIP performs synchronously, so no
// pinned staging buffer is allocated either.
//
// Nothing in the scratch needs clearing: every kernel writes what a later one reads
// (the dQ kernel writes -D and -LSE / scale of every row before the dK/dV kernel reads
// them; split-mode slices are written in full), and the lists are copied per call.
// Every call on one device shares its array, so calls that overlap on one GPU (on
// different streams, or from different host threads) race; a caller runs them one
// after another.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "../../include/dkv.h"
#include "dkv_internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void *g_scratch[kMaxDevices] = {};

// The current device's address of `scratch`, looked up on the first call on a device.
dkv_status scratch_ptr(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return dkv::report(DKV_ERR_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices) return dkv::report(DKV_ERR_UNSUPPORTED, "device index out of range");
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      char msg[160];
      std::snprintf(msg, sizeof msg, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
      return dkv::report(DKV_ERR_HIP, msg);
    }
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return DKV_OK;
}

}  // namespace

extern "C" dkv_status dkv_bwd_noalloc(const dkv_params *p, const void *q_resp, const void *k_p,
                                      const void *v_p, const void *k_r, const void *v_r,
                                      const void *o_r, const float *lse_r, const void *dout_r,
                                      void *dq_r, void *dk_r, void *dv_r, float *acc_dk_p,
                                      float *acc_dv_p, int acc_flags, void *dk_p, void *dv_p,
                                      hipStream_t stream) {
  const int call = (acc_flags & DKV_ACC_SPLIT) ? DKV_CALL_BWD_SPLIT : DKV_CALL_BWD;
  const size_t need = dkv_workspace_size(p, call);
  if (need == (size_t)-1)   // invalid parameters: the full call reports why
    return dkv::bwd_call(p, q_resp, k_p, v_p, k_r, v_r, o_r, lse_r, dout_r, dq_r, dk_r, dv_r,
                         acc_dk_p, acc_dv_p, acc_flags, dk_p, dv_p, nullptr, 0, stream, true);
  if (need > kScratchBytes) {
    char msg[200];
    std::snprintf(msg, sizeof msg,
                  "dkv_bwd_noalloc: this call needs %zu bytes of scratch; the entry point "
                  "holds %zu (use dkv_bwd with a workspace)", need, kScratchBytes);
    return dkv::report(DKV_ERR_UNSUPPORTED, msg);
  }
  void *ws = nullptr;
  if (dkv_status st = scratch_ptr(&ws)) return st;
  return dkv::bwd_call(p, q_resp, k_p, v_p, k_r, v_r, o_r, lse_r, dout_r, dq_r, dk_r, dv_r,
                       acc_dk_p, acc_dv_p, acc_flags, dk_p, dv_p, ws, kScratchBytes, stream, true);
}
