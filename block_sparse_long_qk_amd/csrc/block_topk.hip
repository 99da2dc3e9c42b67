// Index Branch, part 2: exp-free block top-k with the forced local block.
//
// Page "MiniMax 发布 MSA 稀疏注意力方法，开源推理内核并推出 MiniMax-M3 模型":
// section 两个分支如何工作 (top-k blocks per query and group; the block holding
// the query is always included) and section 内核协同设计 (softmax preserves the
// order, so the selection runs on the raw scores with no max, exp or sum).
//
// One wavefront per (sequence, group, query) row; the waves stay resident and
// walk the rows, the next row's scores loading while the current one is
// selected.  Scores are compared as fp32 values (-0 equals +0; lanes and slots
// without a candidate hold -inf, and pooled scores are finite).  Selection:
//   0. the row's candidate scores (blocks t < l, l = the local block; block t
//      = lane + 64 j) are loaded into registers through a buffer descriptor
//      whose range is the row;
//   1. each lane takes the max of its share of the row, and tau is a value
//      that at least k-1 lane maxima reach: for k-1 <= 16 and rows held in
//      registers the smallest over the
//      four rows of 16 lanes of each row's ceil((k-1)/4)-th largest (sorts of
//      16 lanes, DPP moves only), else the (k-1)-th largest of all 64 (a
//      sorting network, mostly DPP moves).  At least k-1 scores of the row are
//      >= tau, and for score rows of any shape only a few dozen more;
//   2. the scores >= tau are compacted into LDS in ascending block order with
//      their block ids, one per lane, and T, the (k-1)-th largest of them, is
//      read off a sorted copy (16, 32 or 64 lanes, as many as they need);
//      should more than 64 pass tau (many equal scores), T comes from a bitwise
//      search over the whole row instead;
//   3. the blocks scoring > T, and the lowest-indexed blocks scoring == T until
//      k-1 are taken (equal scores go to the lower index), are written in
//      ascending order (ballot ranks), then the local block.
#include <algorithm>
#include <type_traits>

#include "launch.h"

namespace msa {
namespace {

// Order-preserving unsigned key of a score (the bitwise search of rows with
// many equal scores): -0 + 0 = +0 folds the signed zeros, then negative scores
// have all bits flipped and positive ones the sign bit set.
__device__ __forceinline__ uint32_t sel_key(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

// Partner values for the sorting network, each lane getting lane ^ M's value.
// Within a row of 16 lanes they are DPP moves (no LDS): ^1, ^2 and ^3 are
// quad permutes, ^7 and ^15 the half-row and row mirrors, ^8 a rotate of the
// row by 8, ^4 the half-row mirror followed by the quad flip.  Across rows:
// ^16 and ^31 by ds_swizzle (xor within 32 lanes), ^63 by ds_bpermute.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
template <int M>
__device__ __forceinline__ float xor_lane(float v) {
  if constexpr (M == 1) return dpp_f32<0xB1>(v);                  // quad_perm [1, 0, 3, 2]
  else if constexpr (M == 2) return dpp_f32<0x4E>(v);             // quad_perm [2, 3, 0, 1]
  else if constexpr (M == 3) return dpp_f32<0x1B>(v);             // quad_perm [3, 2, 1, 0]
  else if constexpr (M == 4) return dpp_f32<0x1B>(dpp_f32<0x141>(v));
  else if constexpr (M == 7) return dpp_f32<0x141>(v);            // row_half_mirror
  else if constexpr (M == 8) return dpp_f32<0x128>(v);            // row_ror:8
  else if constexpr (M == 15) return dpp_f32<0x140>(v);           // row_mirror
  else if constexpr (M == 16)
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
  else if constexpr (M == 31)
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x7C1F));
  else return __shfl_xor(v, M, 64);
}

// Compare-exchange with lane ^ M: the lane whose `LOWBIT` is clear keeps the smaller.
template <int M, int LOWBIT>
__device__ __forceinline__ float cmpx(float x, int lane) {
  const float y = xor_lane<M>(x);
  return (lane & LOWBIT) == 0 ? fminf(x, y) : fmaxf(x, y);
}
template <int S>
__device__ __forceinline__ float half_clean(float x, int lane) {  // xor partners S, S/2, ..., 1
  if constexpr (S == 0) {
    return x;
  } else {
    x = cmpx<S, S>(x, lane);
    return half_clean<S / 2>(x, lane);
  }
}
template <int SIZE>
__device__ __forceinline__ float merge_level(float x, int lane) {
  x = cmpx<SIZE - 1, SIZE / 2>(x, lane);  // flip: lane i against SIZE-1-i of its block
  return half_clean<SIZE / 4>(x, lane);
}

// Ascending sort of one value per lane over blocks of N lanes (16, 32 or 64):
// a bitonic network in its flip form (each merge level starts by comparing
// lane i with the mirrored lane of its block, then halves with xor partners),
// so that all but three of the 64-lane network's 21 exchange steps, and all of
// the 16-lane one's, are DPP moves.
template <int N>
__device__ __forceinline__ float sort_lanes(float x, int lane) {
  x = merge_level<16>(merge_level<8>(merge_level<4>(merge_level<2>(x, lane), lane), lane), lane);
  if constexpr (N >= 32) x = merge_level<32>(x, lane);
  if constexpr (N >= 64) x = merge_level<64>(x, lane);
  return x;
}

__device__ __forceinline__ float lane_f32(float x, int src) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), src));
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Number of the wave's lanes where pred holds (a scalar).
__device__ __forceinline__ int count(bool pred) { return __popcll(__ballot(pred)); }

// base + the number of set bits of m below this lane (two VALU ops).
__device__ __forceinline__ int prefix(uint64_t m, int base = 0) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, (uint32_t)base));
}

// PER > 0: a row's candidates (at most 64 * PER) are loaded once into
// registers, the next row's while the current one is selected; PER == 0 (rows
// beyond 2048 blocks): each of the two passes over the row streams it, eight
// loads in flight (the second pass mostly from L2).
template <int PER, bool VL>
__global__ __launch_bounds__(256) void k_block_topk(const float* __restrict__ pooled, int32_t* __restrict__ out,
                                                    Dims D, int nrows) {
  __shared__ uint2 cand[4][64];  // (score bits, block) of the row's scores >= tau
  // the wave index as a uniform value, so that the rows' buffer descriptors
  // live in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int stride = gridDim.x * 4;
  const float NEG_INF = -__builtin_huge_valf();
  const int k = D.k, kk = k - 1;  // kk blocks to pick among a row's `local` candidates
  constexpr int NREG = PER > 0 ? PER : 1;

  // A row (r < nrows: the launch's rows number below 2^31): its local block
  // (-1: nothing to do) and the descriptor of its candidate scores (offsets
  // past the candidates read 0 and never leave them).
  struct Row {
    int r, local;
    __amdgpu_buffer_rsrc_t rs;
  };
  auto row_at = [&](int r) {
    Row x;
    x.r = r;
    x.local = -1;
    if (r < nrows) {
      const int i = r % D.n_q;
      if constexpr (VL) {
        const int b = r / (D.h_kv * D.n_q);
        if (i < seq_nq(D, b)) x.local = (int)((seq_offset(D, b) + i) / kBk);  // rows past a sequence's queries: none
      } else {
        x.local = (int)((D.offset + i) / kBk);
      }
    }
    x.rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(pooled + (int64_t)r * D.n_blk), (short)0,
                                             max(x.local, 0) * 4, kRawBufferFlags);
    return x;
  };
  auto load = [&](const Row& x, int j) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(x.rs, 4 * lane + 256 * j, 0, 0));
  };
  // registers of a row's scores: issued now, used later
  auto fetch = [&](const Row& x, float (&v)[NREG]) {
    if constexpr (PER > 0) {
      const int nj = (x.local + 63) >> 6;
#pragma unroll
      for (int j = 0; j < PER; ++j)
        if (j < nj) v[j] = load(x, j);
    }
  };

  Row cur = row_at(blockIdx.x * 4 + wave);
  float vc[NREG];
  fetch(cur, vc);
  while (cur.r < nrows) {
    const Row nxt = row_at(cur.r + stride);
    float vn[NREG];
    fetch(nxt, vn);
    const int local = cur.local;
    int32_t* dst = out + (int64_t)cur.r * k;
    if (local < 0) {
      // not a row of this batch
    } else if (local + 1 <= k) {  // every visible block is kept
      for (int s = lane; s < k; s += 64) dst[s] = s <= local ? s : -1;
    } else if (kk == 0) {
      if (lane == 0) dst[0] = local;
    } else {
      const int nj = (local + 63) >> 6;  // score slots in use (uniform)
      // f(j, score of block lane + 64 j) for j = 0 .. nj-1, in order; only the
      // last slot can reach past the candidates
      if constexpr (PER > 0) {  // the last slot's scores past the candidates become -inf, in place
#pragma unroll
        for (int j = 0; j < PER; ++j)
          if (j == nj - 1) vc[j] = lane + 64 * j < local ? vc[j] : NEG_INF;
      }
      auto each_score = [&](auto&& f) {
        if constexpr (PER > 0) {
#pragma unroll
          for (int j = 0; j < PER; ++j)
            if (j < nj) f(j, vc[j]);
        } else {
          for (int j0 = 0; j0 < nj; j0 += 8) {  // eight loads in flight per step
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = load(cur, j0 + u);
#pragma unroll
            for (int u = 0; u < 8; ++u)
              if (j0 + u < nj) f(j0 + u, lane + 64 * (j0 + u) < local ? v[u] : NEG_INF);
          }
        }
      };

      // 1. tau: for kk <= 16, the smallest over the four rows of 16 lanes of
      // the row's m-th largest lane maximum (m = ceil(kk / 4)): 4 m >= kk lane
      // maxima are >= tau, and the 16-lane sorts are DPP moves only; else the
      // kk-th largest lane maximum
      float mx = NEG_INF;
      each_score([&](int, float c) { mx = fmaxf(mx, c); });
      float tau;
      if (PER > 0 && kk <= 16) {  // rows in registers (streamed rows keep the tighter tau: fewer candidates)
        const float srt = sort_lanes<16>(mx, lane);
        const int pos = 16 - ((kk + 3) >> 2);
        tau = fminf(fminf(lane_f32(srt, pos), lane_f32(srt, 16 + pos)),
                    fminf(lane_f32(srt, 32 + pos), lane_f32(srt, 48 + pos)));
      } else {
        tau = lane_f32(sort_lanes<64>(mx, lane), 64 - kk);
      }

      // 2. scores >= tau, compacted in ascending block order (slot 63 takes
      // the overflow of a row with more than 64, whose list is not used)
      int total = 0;
      each_score([&](int j, float c) {
        const bool take = c >= tau;
        const uint64_t m = __ballot(take);
        if (m) {
          const int slot = prefix(m, total);
          if (take) cand[wave][slot < 63 ? slot : 63] = make_uint2(__float_as_uint(c), (uint32_t)(lane + 64 * j));
          total += __popcll(m);
        }
      });
      if (total <= 64) {
        wave_lds_sync();
        const bool have = lane < total;
        const uint2 e = cand[wave][lane];
        const float c = have ? __uint_as_float(e.x) : NEG_INF;
        // T from a sorted copy of the candidates: a network over the first 16
        // or 32 lanes when they hold them all (uniform branch on total)
        float thr;
        if (total <= 16 && kk <= 16)
          thr = lane_f32(sort_lanes<16>(c, lane), 16 - kk);
        else if (total <= 32 && kk <= 32)
          thr = lane_f32(sort_lanes<32>(c, lane), 32 - kk);
        else
          thr = lane_f32(sort_lanes<64>(c, lane), 64 - kk);
        // 3. emit: scores > T, then scores == T in block order until kk
        const uint64_t meq = __ballot(have && c == thr);
        const int need_eq = kk - count(have && c > thr);
        const bool take = have && (c > thr || (c == thr && prefix(meq) < need_eq));
        const uint64_t m = __ballot(take);
        if (take) dst[prefix(m)] = (int)e.y;
      } else {
        // many equal scores: T = the largest key x with #{keys >= x} >= kk, bit by bit
        uint32_t thr = 0;
        for (int bit = 31; bit >= 0; --bit) {
          const uint32_t trial = thr | (1u << bit);
          int n = 0;
          each_score([&](int, float c) { n += count(sel_key(c) >= trial); });
          if (n >= kk) thr = trial;
        }
        int n_gt = 0;
        each_score([&](int, float c) { n_gt += count(sel_key(c) > thr); });
        const int need_eq = kk - n_gt;  // >= 1 keys equal to T are taken
        int base = 0, eq_seen = 0;
        each_score([&](int j, float c) {
          const uint32_t u = sel_key(c);
          const bool eq = u == thr;
          const uint64_t meq = __ballot(eq);
          const bool take = u > thr || (eq && prefix(meq, eq_seen) < need_eq);
          const uint64_t m = __ballot(take);
          if (take) dst[prefix(m, base)] = lane + 64 * j;
          base += __popcll(m);
          eq_seen += __popcll(meq);
        });
      }
      if (lane == 0) dst[kk] = local;
      wave_lds_sync();  // the list is read before the next row overwrites it
    }
    cur = nxt;
#pragma unroll
    for (int j = 0; j < NREG; ++j) vc[j] = vn[j];
  }
}

}  // namespace

hipError_t launch_block_topk(const float* pooled, int32_t* block_idx, const Dims& D, hipStream_t stream) {
  const int64_t nrows = (int64_t)D.B * D.h_kv * D.n_q;
  // resident waves that walk the rows: up to 8 workgroups of 4 waves per CU
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus = n;
  }
  const dim3 grid((unsigned)std::min<int64_t>((nrows + 3) / 4, (int64_t)cus * 8)), block(256);
  const int n = (int)nrows;  // below 2^31 (the problem's row count is checked on the host)
  // scores per lane for the longest row (rows are at most n_blk - 1 candidates)
  const int per = (D.n_blk + 63) / 64;
  auto go = [&](auto per_c, auto vl) {
    hipLaunchKernelGGL((k_block_topk<decltype(per_c)::value, decltype(vl)::value>), grid, block, 0, stream, pooled,
                       block_idx, D, n);
    mark("k_block_topk", stream);
  };
  auto pick = [&](auto vl) {
    if (per <= 4) go(std::integral_constant<int, 4>{}, vl);
    else if (per <= 8) go(std::integral_constant<int, 8>{}, vl);
    else if (per <= 16) go(std::integral_constant<int, 16>{}, vl);
    else if (per <= 32) go(std::integral_constant<int, 32>{}, vl);
    else go(std::integral_constant<int, 0>{}, vl);
  };
  if (dims_varlen(D)) pick(std::true_type{}); else pick(std::false_type{});
  return hipGetLastError();
}

}  // namespace msa
