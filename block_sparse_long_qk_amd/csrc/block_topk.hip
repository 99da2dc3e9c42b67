// Index Branch, part 2: exp-free block top-k with the forced local block.
//
// Page "MiniMax 发布 MSA 稀疏注意力方法，开源推理内核并推出 MiniMax-M3 模型":
// section 两个分支如何工作 (top-k blocks per query and group; the block holding
// the query is always included) and section 内核协同设计 (softmax preserves the
// order, so the selection runs on the raw scores with no max, exp or sum).
//
// One wavefront per (sequence, group, query) row.  Every candidate block t < l
// (l = the local block) is turned into a 64-bit key
//     (order-preserving bits of the fp32 score, -0 folded onto +0) << 32 | ~t
// so a single unsigned compare ranks by (score desc, index asc) and all keys of
// a row are distinct.  Selection:
//   0. rows of up to 2048 blocks are loaded into registers once;
//   1. each lane takes the max key of its strided share of the row;
//   2. a bitonic sort of the 64 lane maxima gives tau, the (k-1)-th largest of
//      them; at least k-1 keys of the row are >= tau, and for score rows of any
//      shape only a handful more;
//   3. the keys >= tau are compacted into LDS (one per lane) and sorted: the
//      (k-1)-th largest of them is the exact threshold; should more than 64 pass
//      tau, an exact bitwise threshold search over the whole row takes over;
//   4. the selected blocks are emitted in ascending order with ballots (rank =
//      number of selected blocks with a smaller index), then the local block.
#include "launch.h"

namespace msa {
namespace {

__device__ __forceinline__ uint64_t sel_key(float f, int t) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;                       // -0 ranks as +0
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);     // order-preserving
  return ((uint64_t)u << 32) | (uint32_t)(~(uint32_t)t);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t x, int m) {
  const uint32_t lo = __shfl_xor((uint32_t)x, m, 64);
  const uint32_t hi = __shfl_xor((uint32_t)(x >> 32), m, 64);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t shfl_u64(uint64_t x, int src) {
  const uint32_t lo = __shfl((uint32_t)x, src, 64);
  const uint32_t hi = __shfl((uint32_t)(x >> 32), src, 64);
  return ((uint64_t)hi << 32) | lo;
}

// Bitonic sort of one value per lane, ascending over lanes 0..63.
__device__ __forceinline__ uint64_t wave_sort_asc(uint64_t x, int lane) {
#pragma unroll
  for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const uint64_t y = shfl_xor_u64(x, stride);
      const bool asc = (lane & size) == 0;
      const bool lower = (lane & stride) == 0;
      const uint64_t mn = x < y ? x : y, mx = x < y ? y : x;
      x = (lower == asc) ? mn : mx;
    }
  }
  return x;
}

__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// PER > 0: the row's candidates (at most 64*PER) are loaded once into
// registers and every pass runs on them; PER == 0: passes re-read the row.
template <int PER>
__global__ __launch_bounds__(256) void k_block_topk(const float* __restrict__ pooled, int32_t* __restrict__ out,
                                                    Dims D, int64_t nrows) {
  __shared__ uint64_t cand[4][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + wave;
  if (row >= nrows) return;  // whole wave; no workgroup barrier below
  const int i = (int)(row % D.n_q);
  const int b = (int)(row / ((int64_t)D.h_kv * D.n_q));
  if (i >= seq_nq(D, b)) return;  // a row past this sequence's queries (variable lengths)
  const int local = (int)((seq_offset(D, b) + i) / kBk);
  const float* src = pooled + row * D.n_blk;
  int32_t* dst = out + row * D.k;
  const int k = D.k;

  if (local + 1 <= k) {  // every visible block is kept
    for (int s = lane; s < k; s += 64) dst[s] = s <= local ? s : -1;
    return;
  }
  const int kk = k - 1;  // blocks to pick among the `local` candidates
  if (kk == 0) {
    if (lane == 0) dst[0] = local;
    return;
  }

  constexpr int NREG = PER > 0 ? PER : 1;
  uint64_t reg[NREG];  // keys of t = lane + 64*j (0 = no candidate)
  if constexpr (PER > 0) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int t = lane + 64 * j;
      reg[j] = t < local ? sel_key(src[t], t) : 0;
    }
  }
  auto key_at = [&](int j, int t) -> uint64_t {
    if constexpr (PER > 0) return reg[j];
    else return t < local ? sel_key(src[t], t) : 0;
  };
  const int nj = PER > 0 ? PER : (local + 63) / 64;

  // 1. lane maxima
  uint64_t mx = 0;
  for (int j = 0; j < nj; ++j) {
    const uint64_t c = key_at(j, lane + 64 * j);
    mx = c > mx ? c : mx;
  }
  // 2. tau = kk-th largest lane maximum (lanes without candidates hold 0)
  const uint64_t tau = shfl_u64(wave_sort_asc(mx, lane), 64 - kk);

  // 3. compact the keys >= tau and find the exact kk-th largest key
  int mine = 0;
  for (int j = 0; j < nj; ++j) mine += key_at(j, lane + 64 * j) >= tau;
  int incl = mine;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  const int total = __shfl(incl, 63, 64);
  uint64_t thr;
  if (total <= 64) {
    int at = incl - mine;
    for (int j = 0; j < nj; ++j) {
      const uint64_t c = key_at(j, lane + 64 * j);
      if (c >= tau) cand[wave][at++] = c;
    }
    wave_lds_sync();
    const uint64_t mine_c = lane < total ? cand[wave][lane] : 0;
    thr = shfl_u64(wave_sort_asc(mine_c, lane), 64 - kk);
  } else {
    // exact threshold: the largest key x with #{keys >= x} >= kk, bit by bit
    uint64_t prefix = 0;
    for (int bit = 63; bit >= 0; --bit) {
      const uint64_t trial = prefix | (1ull << bit);
      int c = 0;
      for (int j = 0; j < nj; ++j) c += key_at(j, lane + 64 * j) >= trial;
      if (wave_sum(c) >= kk) prefix = trial;
    }
    thr = prefix;
  }

  // 4. ascending output: rank by ballot over the strided slots
  int base = 0;
  for (int j = 0; j < nj; ++j) {
    const int t = lane + 64 * j;
    const bool take = t < local && key_at(j, t) >= thr;
    const uint64_t m = __ballot(take);
    if (take) dst[base + __popcll(m & ((1ull << lane) - 1ull))] = t;
    base += __popcll(m);
  }
  if (lane == 0) dst[kk] = local;
}

}  // namespace

hipError_t launch_block_topk(const float* pooled, int32_t* block_idx, const Dims& D, hipStream_t stream) {
  const int64_t nrows = (int64_t)D.B * D.h_kv * D.n_q;
  const int64_t blocks = (nrows + 3) / 4;
  if (D.n_blk <= 64 * 16)
    hipLaunchKernelGGL(k_block_topk<16>, dim3((unsigned)blocks), dim3(256), 0, stream, pooled, block_idx, D, nrows);
  else if (D.n_blk <= 64 * 32)
    hipLaunchKernelGGL(k_block_topk<32>, dim3((unsigned)blocks), dim3(256), 0, stream, pooled, block_idx, D, nrows);
  else
    hipLaunchKernelGGL(k_block_topk<0>, dim3((unsigned)blocks), dim3(256), 0, stream, pooled, block_idx, D, nrows);
  return hipGetLastError();
}

}  // namespace msa
