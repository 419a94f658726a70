// csa_index_topk_noalloc: the index + top-k entry point without a caller
// workspace, for callers that cannot allocate device memory (code under HIP
// graph capture, serving loops that forbid hipMalloc).  Its workspace is a
// fixed device array of CSA_NOALLOC_SCRATCH_BYTES; calls run in query blocks
// sized to fit it.
#include <stdint.h>

#include <mutex>

#include <hip/hip_runtime.h>

#include "api_internal.hpp"
#include "csa.h"

#define CSA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

constexpr size_t kScratchBytes = CSA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

// One copy per GPU, held until the process ends.  In host code `scratch`
// names a host-side stand-in, never the device memory: kernels and fills
// take the address hipGetSymbolAddress returns on the current device, looked
// up once per device and kept in g_scratch.
static __device__ __attribute__((aligned(256))) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];

// The current device's scratch address; CSA_EHIP when it cannot be found.
int scratch_address(char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CSA_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return CSA_EHIP;
    g_scratch[dev] = p;
  }
  *out = (char*)g_scratch[dev];
  return CSA_OK;
}

// Zero n 32-bit words: a kernel rather than hipMemsetAsync, so the call may
// be recorded into a HIP graph.
__global__ void __launch_bounds__(256) zero_words_kernel(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = 0u;
}

}  // namespace

CSA_EXPORT int csa_index_topk_noalloc(const CsaIndexArgs* a, void* stream) {
  int st = csa::api::check_index(a);
  if (st) return st;
  const csa::api::IndexPlan p = csa::api::plan_index(a, (int64_t)kScratchBytes);
  if (p.n_qb < 1 || p.total > kScratchBytes) return CSA_ESCRATCH;
  char* ws = nullptr;
  st = scratch_address(&ws);
  if (st) return st;
  // The histograms are the only part of the workspace that must start at
  // zero; the previous call on this GPU (or a failed one) may have left them
  // in any state.
  const size_t words = (p.off_state - p.off_hist) / 4;
  const size_t blocks = (words + 255) / 256;
  zero_words_kernel<<<(unsigned)(blocks < 1024 ? blocks : 1024), 256, 0, (hipStream_t)stream>>>(
      (uint32_t*)(ws + p.off_hist), words);
  if (hipGetLastError() != hipSuccess) return CSA_EHIP;
  return csa::api::run_index(a, p, ws, stream);
}
