// static_scratch.hip -- kdn_scan_fwd_static: the scan with the library's own
// scratch memory instead of a caller workspace, for callers that cannot
// allocate (code under graph capture, serving loops, allocation-free harnesses).
//
// The scratch is one file-scope device array. In host code its name is only a
// host-side stand-in, so it is never passed to a kernel or a copy: the device
// address of each GPU's copy is looked up once per device with
// hipGetSymbolAddress (that device current) and kept, and only that address
// is handed to the kernels, as the workspace argument of the ordinary entry.
#include "../../include/kdn.h"

#include <hip/hip_runtime.h>

#include <mutex>

#include "kdn_internal.h"

#define KDN_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

constexpr size_t kScratchBytes = KDN_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current GPU's scratch array (looked up on first use).
// Returns KDN_OK, a positive hipError_t, or KDN_ERR_UNSUPPORTED for a device
// index past the table.
int current_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return static_cast<int>(e);
  if (dev < 0 || dev >= kMaxDevices) return KDN_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return static_cast<int>(e);
    if (p == nullptr) return static_cast<int>(hipErrorInvalidSymbol);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return KDN_OK;
}

}  // namespace

KDN_EXPORT int kdn_scan_fwd_static(const void* q, const void* k, const void* v, int in_dtype,
                                   const float* alpha, const float* beta, const float* r,
                                   const float* cov_in, float* cov_out, float q_noise_var,
                                   const float* state_in, float* state_out, void* o,
                                   int out_dtype, float* m, int score_kind, int B, int H, int L,
                                   int d_k, int d_v, int chunk, int mode, int resid,
                                   void* stream) {
  // every argument check first: no HIP call for a rejected call
  const int st = kdn::scan_args_status(KDN_PHASE_ALL, q, k, v, in_dtype, beta, cov_in,
                                       q_noise_var, o, out_dtype, m, score_kind, B, H, L, d_k,
                                       d_v, chunk, mode, resid);
  if (st != KDN_OK) return st;
  const size_t need =
      kdn_scan_workspace_size(B, H, L, d_k, d_v, chunk, mode, in_dtype, m != nullptr ? 1 : 0);
  if (need > kScratchBytes) return KDN_ERR_SCRATCH_LIMIT;
  void* ws = nullptr;
  const int sp = current_scratch(&ws);
  if (sp != KDN_OK) return sp;
  return kdn_scan_fwd(q, k, v, in_dtype, alpha, beta, r, cov_in, cov_out, q_noise_var, state_in,
                      state_out, o, out_dtype, m, score_kind, B, H, L, d_k, d_v, chunk, mode,
                      resid, ws, kScratchBytes, stream);
}
