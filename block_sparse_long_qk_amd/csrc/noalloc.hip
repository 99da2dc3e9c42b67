// msa_forward for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops): the workspace is a fixed array in the
// library's own device memory instead of a caller's buffer.
//
// `scratch` is a file-scope device array; every GPU the library runs on holds
// its own copy, at its own address, until the process ends.  Host code never
// uses the array's name as an address (on the host it is only a stand-in):
// the address of the current device's copy is looked up once per device with
// hipGetSymbolAddress and kept, and that pointer is what the kernels get, as
// the workspace argument of msa_forward.  The forward kernels write every
// workspace byte they later read, so the array needs no clearing between
// calls.  Calls on one GPU share its array: two calls that overlap in time on
// one GPU (on different streams) race on it.
#include <mutex>

#include <hip/hip_runtime.h>

#include "../../include/msa.h"

namespace {

constexpr size_t kScratchBytes = size_t(128) << 20;  // MSA_NOALLOC_SCRATCH_BYTES
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// The current device's copy of `scratch` (resolved on the first call per device).
msa_status scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MSA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MSA_ERR_HIP;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return MSA_OK;
}

}  // namespace

static_assert(kScratchBytes == MSA_NOALLOC_SCRATCH_BYTES, "the header states the scratch size");

extern "C" msa_status msa_forward_noalloc(const msa_problem* p, const void* q, const void* k, const void* v,
                                          const void* index_q, const void* index_k, void* out, int32_t* block_idx,
                                          float* lse, hipStream_t stream) {
  size_t need = 0;
  const msa_status st = msa_workspace_size(p, MSA_OP_FORWARD, &need);  // validates p; host only
  if (st != MSA_OK) return st;
  if (need > kScratchBytes) return MSA_ERR_WORKSPACE_TOO_SMALL;
  void* ws = nullptr;
  const msa_status sp = scratch_ptr(&ws);
  if (sp != MSA_OK) return sp;
  return msa_forward(p, q, k, v, index_q, index_k, out, block_idx, lse, ws, kScratchBytes, stream);
}
