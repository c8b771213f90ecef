// butler_select_attend_noalloc: butler_select_attend for callers that cannot allocate
// (code under HIP graph capture, serving loops that forbid hipMalloc).  Its workspace is a
// file-scope device array of fixed size instead of a caller buffer; the library holds one
// copy per GPU until the process ends.
//
// On the host the array's name is only a stand-in: the device address of each GPU's copy
// is looked up once per device (hipGetSymbolAddress, with that device current) and that
// address is what the kernels are given.  Every call on a GPU shares that GPU's copy, so
// calls that overlap on one GPU race; each call first clears, on its own stream and with a
// kernel (a captured graph must not hold memset nodes), the part of the array whose
// contents must start at zero.
#include <mutex>

#include "../../include/butler.h"
#include "common.h"
#include "kernels.h"

namespace butler {
namespace {

constexpr size_t kScratchBytes = BUTLER_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "whole 256-byte lines");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of each GPU's copy, once looked up

// The current device's copy of the array.
int scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return BUTLER_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return BUTLER_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return BUTLER_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return BUTLER_OK;
}

__global__ __launch_bounds__(256) void scratch_clear_kernel(uint4* __restrict__ p,
                                                            long long n16) {
  const long long stride = (long long)gridDim.x * 256;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

}  // namespace
}  // namespace butler

using namespace butler;

extern "C" int butler_select_attend_noalloc(void* stream, int dtype, const float* scores,
                                            uint32_t* radix_hist, int budget_num,
                                            int budget_den, int n_sink, int n_window,
                                            int budget_excludes_forced, int32_t* idx,
                                            int32_t* count, const void* q, const void* k_cache,
                                            const void* v_cache, float* out, int B, int Hq,
                                            int Hkv, int sel_group, int D, int L, int L_cap,
                                            int cap, float softmax_scale) {
  SelectAttendArgs a{dtype, scores, radix_hist, budget_num, budget_den, n_sink, n_window,
                     budget_excludes_forced, idx, count, q, k_cache, v_cache, out, B, Hq, Hkv,
                     sel_group, D, L, L_cap, cap, softmax_scale};
  SelectAttendPlan plan;
  int rc = select_attend_plan(a, &plan);
  if (rc != BUTLER_OK) return rc;
  if (plan.need > kScratchBytes) return BUTLER_ERR_WORKSPACE;   // beyond the fixed array
  rc = select_attend_check_pointers(a);
  if (rc != BUTLER_OK) return rc;
  void* ws = nullptr;
  rc = scratch_ptr(&ws);
  if (rc != BUTLER_OK) return rc;
  hipStream_t s = (hipStream_t)stream;
  // the selection state (first-digit and coarse histograms, call counters) starts at zero
  const long long n16 = (long long)(select_state_bytes(plan.rows) / 16);
  const unsigned blocks = (unsigned)((n16 + 255) / 256 < 1024 ? (n16 + 255) / 256 : 1024);
  hipLaunchKernelGGL(scratch_clear_kernel, dim3(blocks), dim3(256), 0, s, (uint4*)ws, n16);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return finish_call(s, e);
  return finish_call(s, select_attend_launch(s, a, plan, ws));
}
