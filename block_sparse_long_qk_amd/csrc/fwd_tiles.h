// Pieces of the four-wave KV-outer tile kernels (the forward attention and the
// KL pass): query rows held in VGPRs, runs of tiles claimed per XCD, and the
// LDS-only workgroup barrier.
#pragma once

#include "attn_tiles.h"

namespace msa {
namespace {

// The four-wave tile workgroups (128 query rows per tile) hold only one block
// in LDS (the forward: K and V, 65 KB; the KL pass: K and the index keys);
// each wave keeps its 32 query rows in VGPRs.  Two such workgroups fill a CU.
constexpr int kFWaves = 4;
constexpr int kFThreads = 64 * kFWaves;
constexpr int kFRows = 32 * kFWaves;
constexpr int kFRun = 16;  // most tiles per claimed run

// Lane (column, half) of a wave's MFMA operand for query row `row`: dims
// 16 ks + 8 half .. + 7 of k-step ks, the order qk_block reads from LDS.
__device__ __forceinline__ void load_q(const uint16_t* row, int half, uint4 (&qf)[8]) {
  const uint16_t* p = row + 8 * half;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) qf[ks] = *reinterpret_cast<const uint4*>(p + 16 * ks);
}

// Dynamic runs.  The tile range [0, total) is cut into kXcds slices; slice x
// is first drained by the workgroups of XCD x (workgroup w runs on XCD
// w % kXcds), which claim runs of consecutive tiles from the slice's
// counter, so consecutive tiles (one K/V block as a rule) stay on one XCD's
// L2.  A run is kFRun tiles, or fewer when the grid would otherwise get under
// four runs per workgroup (short tile lists: a chunk of a long context).  A
// workgroup whose slice is empty moves on to the next slices in turn.
// Workgroups that start late, or share their CU with other work, simply
// claim fewer runs.  Only thread 0 of a workgroup uses it.
struct RunQueue {
  int32_t* ctr;
  int total, len, slice, left;  // len: tiles per run; left: slices not yet found empty
  int pend;                // claimed run of `slice`, not yet resolved
  __device__ void init(int32_t* c, int tot) {
    ctr = c;
    total = tot;
    len = max(1, min(kFRun, tot / (int)(gridDim.x * 4)));
    slice = blockIdx.x % kXcds;
    left = kXcds;
    pend = 0;
  }
  __device__ int2 range(int s, int run) const {
    const int64_t lo = (int64_t)total * s / kXcds, hi = (int64_t)total * (s + 1) / kXcds;
    const int64_t st = lo + (int64_t)run * len;
    if (st >= hi) return make_int2(-1, -1);
    return make_int2((int)st, (int)min<int64_t>(st + len, hi));
  }
  __device__ int2 claim() {  // waits for each counter it reads
    while (left > 0) {
      const int2 r = range(slice, atomicAdd(&ctr[slice], 1));
      if (r.x >= 0) return r;
      slice = (slice + 1) % kXcds;
      --left;
    }
    return make_int2(-1, -1);
  }
  __device__ void prefetch() {  // a claim whose result is looked at later
    if (left > 0) pend = atomicAdd(&ctr[slice], 1);
  }
  __device__ int2 resolve() {
    if (left <= 0) return make_int2(-1, -1);
    const int2 r = range(slice, pend);
    if (r.x >= 0) return r;
    slice = (slice + 1) % kXcds;
    --left;
    return claim();
  }
};

__device__ __forceinline__ int2 uniform2(int2 x) {
  return make_int2(__builtin_amdgcn_readfirstlane(x.x), __builtin_amdgcn_readfirstlane(x.y));
}

// Workgroup barrier for LDS traffic only: this wave's LDS accesses complete,
// then s_barrier.  Unlike __syncthreads(), it does not fence global memory,
// which would wait for every outstanding global load and store (the next
// tile's query rows, the partials just stored).  Direct global-to-LDS loads
// are waited for separately (vmcnt) before such a barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace
}  // namespace msa
