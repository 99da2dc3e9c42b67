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
//   2. a sort of the 64 lane maxima (a bitonic network, mostly DPP moves)
//      gives tau, the (k-1)-th largest of them; at least k-1 keys of the row are
//      >= tau, and for score rows of any shape only a handful more;
//   3. the keys >= tau are compacted into LDS (one per lane) and sorted (over
//      16, 32 or 64 lanes, as many as they need): the (k-1)-th largest of them
//      is the exact threshold; should more than 64 pass tau, an exact bitwise
//      threshold search over the whole row takes over;
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

// Value of lane `src` (uniform) as a uniform.
__device__ __forceinline__ uint64_t lane_u64(uint64_t x, int src) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, src);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), src);
  return ((uint64_t)hi << 32) | lo;
}

// Partner values for the sorting network, each lane getting lane ^ M's value.
// Within a row of 16 lanes they are DPP moves (no LDS): ^1, ^2 and ^3 are
// quad permutes, ^7 and ^15 the half-row and row mirrors, ^8 a rotate of the
// row by 8, ^4 the half-row mirror followed by the quad flip.  Across rows:
// ^16 and ^31 by ds_swizzle (xor within 32 lanes), ^63 by ds_bpermute.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
template <int M>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v) {
  if constexpr (M == 1) return dpp_u32<0xB1>(v);                  // quad_perm [1, 0, 3, 2]
  else if constexpr (M == 2) return dpp_u32<0x4E>(v);             // quad_perm [2, 3, 0, 1]
  else if constexpr (M == 3) return dpp_u32<0x1B>(v);             // quad_perm [3, 2, 1, 0]
  else if constexpr (M == 4) return dpp_u32<0x1B>(dpp_u32<0x141>(v));
  else if constexpr (M == 7) return dpp_u32<0x141>(v);            // row_half_mirror
  else if constexpr (M == 8) return dpp_u32<0x128>(v);            // row_ror:8
  else if constexpr (M == 15) return dpp_u32<0x140>(v);           // row_mirror
  else if constexpr (M == 16) return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F);
  else if constexpr (M == 31) return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x7C1F);
  else return (uint32_t)__shfl_xor((int)v, M, 64);
}
template <int M>
__device__ __forceinline__ uint64_t xor_lane_u64(uint64_t x) {
  return ((uint64_t)xor_lane<M>((uint32_t)(x >> 32)) << 32) | xor_lane<M>((uint32_t)x);
}

// Compare-exchange with lane ^ M: the lane whose `LOWBIT` is clear keeps the smaller.
template <int M, int LOWBIT>
__device__ __forceinline__ uint64_t cmpx(uint64_t x, int lane) {
  const uint64_t y = xor_lane_u64<M>(x);
  const uint64_t mn = x < y ? x : y, mx = x < y ? y : x;
  return (lane & LOWBIT) == 0 ? mn : mx;
}
template <int S>
__device__ __forceinline__ uint64_t half_clean(uint64_t x, int lane) {  // xor partners S, S/2, ..., 1
  if constexpr (S == 0) {
    return x;
  } else {
    x = cmpx<S, S>(x, lane);
    return half_clean<S / 2>(x, lane);
  }
}
template <int SIZE>
__device__ __forceinline__ uint64_t merge_level(uint64_t x, int lane) {
  x = cmpx<SIZE - 1, SIZE / 2>(x, lane);  // flip: lane i against SIZE-1-i of its block
  return half_clean<SIZE / 4>(x, lane);
}

// Sort of one value per lane, ascending over lanes 0..63: a bitonic network
// in its flip form (each merge level starts by comparing lane i with the
// mirrored lane of its block, then halves with xor partners), so that 18 of
// its 21 exchange steps are DPP moves.
__device__ __forceinline__ uint64_t wave_sort_asc(uint64_t x, int lane) {
  x = merge_level<2>(x, lane);
  x = merge_level<4>(x, lane);
  x = merge_level<8>(x, lane);
  x = merge_level<16>(x, lane);
  x = merge_level<32>(x, lane);
  return merge_level<64>(x, lane);
}

// Inclusive prefix sum over the 64 lanes: DPP shifts within rows of 16, then
// the row broadcasts of lanes 15 and 31 (no LDS).
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
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
  const uint64_t tau = lane_u64(wave_sort_asc(mx, lane), 64 - kk);

  // 3. compact the keys >= tau and find the exact kk-th largest key
  int mine = 0;
  for (int j = 0; j < nj; ++j) mine += key_at(j, lane + 64 * j) >= tau;
  const int incl = wave_incl_scan(mine);
  const int total = __builtin_amdgcn_readlane(incl, 63);
  uint64_t thr;
  if (total <= 64) {
    int at = incl - mine;
    for (int j = 0; j < nj; ++j) {
      const uint64_t c = key_at(j, lane + 64 * j);
      if (c >= tau) cand[wave][at++] = c;
    }
    wave_lds_sync();
    const uint64_t mine_c = lane < total ? cand[wave][lane] : 0;
    // the candidates sit in lanes 0 .. total-1: a network over the first 16 or
    // 32 lanes orders them when they fit there (uniform branch on total)
    if (total <= 16 && kk <= 16) {
      const uint64_t x = merge_level<16>(merge_level<8>(merge_level<4>(merge_level<2>(mine_c, lane), lane), lane), lane);
      thr = lane_u64(x, 16 - kk);
    } else if (total <= 32 && kk <= 32) {
      uint64_t x = merge_level<16>(merge_level<8>(merge_level<4>(merge_level<2>(mine_c, lane), lane), lane), lane);
      thr = lane_u64(merge_level<32>(x, lane), 32 - kk);
    } else {
      thr = lane_u64(wave_sort_asc(mine_c, lane), 64 - kk);
    }
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
