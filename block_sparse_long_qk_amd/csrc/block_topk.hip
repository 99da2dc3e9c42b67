// Index Branch, part 2: exp-free block top-k with the forced local block.
//
// Page "MiniMax 发布 MSA 稀疏注意力方法，开源推理内核并推出 MiniMax-M3 模型":
// section 两个分支如何工作 (top-k blocks per query and group; the block holding
// the query is always included) and section 内核协同设计 (softmax preserves the
// order, so the selection runs on the raw scores with no max, exp or sum).
//
// One wavefront per (sequence, group, query) row for rows of up to 2048
// blocks (k_block_topk), one workgroup of eight waves per row for rows of up
// to 8192 (k_block_topk_wg), one wavefront streaming the row beyond that.  The
// waves stay resident and walk the rows, the next row's scores loading while
// the current one is selected.  Scores are compared as fp32 values (-0 equals
// +0; lanes and slots without a candidate hold -inf, and pooled scores are
// finite).  Selection:
//   0. the row's candidate scores (blocks t < l, l = the local block; block t
//      = lane + 64 j) are loaded into registers through a buffer descriptor
//      whose range is the row (offsets past it read 0);
//   1. each lane takes the max of its share of the row, and tau is a value
//      that at least k-1 lane maxima reach: for k-1 <= 16 and rows held in
//      registers the smallest over the four rows of 16 lanes of each row's
//      ceil((k-1)/4)-th largest (sorts of 16 lanes, DPP moves only), else the
//      (k-1)-th largest of all 64 (a sorting network, mostly DPP moves).  At
//      least k-1 scores of the row are >= tau, and for score rows of any shape
//      only a few dozen more.  Tau is first taken over the registers as
//      loaded; only a row whose tau is not positive has its tail set to -inf
//      and tau taken again;
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
// ^16 and ^31 by ds_swizzle (xor within 32 lanes), ^63 by ds_bpermute (the
// permlane swaps of gfx950 time the same here, with more VALU work).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {  // every lane's source is in its row: no bound control needed
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
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

// Compare-exchange with lane ^ M: the lane whose `LOWBIT` is clear keeps the
// smaller.  One median of three: med3(x, y, -inf) = min(x, y) and
// med3(x, y, +inf) = max(x, y) (no NaNs here), the bound a per-lane constant.
template <int M, int LOWBIT>
__device__ __forceinline__ float cmpx(float x, int lane) {
  const float y = xor_lane<M>(x);
  const float INF = __builtin_huge_valf();
  return __builtin_amdgcn_fmed3f(x, y, (lane & LOWBIT) == 0 ? -INF : INF);
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

// tau from the lane maxima mx, a value that at least kk lane maxima reach.
// kk <= 16 (tau16): the smallest over the four rows of 16 lanes of the row's
// m-th largest lane maximum (m = ceil(kk / 4)): 4 m >= kk lane maxima are >=
// tau, and the 16-lane sorts are DPP moves only.  Else (tau64) the kk-th
// largest lane maximum.
__device__ __forceinline__ float tau16(float mx, int kk, int lane) {
  const float srt = sort_lanes<16>(mx, lane);
  const int pos = 16 - ((kk + 3) >> 2);
  return fminf(fminf(lane_f32(srt, pos), lane_f32(srt, 16 + pos)),
               fminf(lane_f32(srt, 32 + pos), lane_f32(srt, 48 + pos)));
}
__device__ __forceinline__ float tau64(float mx, int kk, int lane) {
  return lane_f32(sort_lanes<64>(mx, lane), 64 - kk);
}

// Steps 2-3 for a row whose scores >= tau (total <= 64 of them, lane i holding
// the i-th in block order: score c, block blk; lanes >= total have = false):
// T, the kk-th largest, from a sorted copy over 16, 32 or 64 lanes (a uniform
// branch on total), then the blocks scoring > T and those == T in block order
// until kk, written to dst in ascending order.
template <bool K16>
__device__ __forceinline__ void emit_from_list(float c, bool have, int blk, int total, int kk, int32_t* dst,
                                               int lane) {
  float thr;
  if (K16 && total <= 16)
    thr = lane_f32(sort_lanes<16>(c, lane), 16 - kk);
  else if (total <= 32 && kk <= 32)
    thr = lane_f32(sort_lanes<32>(c, lane), 32 - kk);
  else
    thr = lane_f32(sort_lanes<64>(c, lane), 64 - kk);
  const uint64_t meq = __ballot(have && c == thr);
  const int need_eq = kk - count(have && c > thr);
  const bool take = have && (c > thr || (c == thr && prefix(meq) < need_eq));
  const uint64_t m = __ballot(take);
  if (take) dst[prefix(m)] = blk;
}

// Rows with more than 64 scores >= tau (many equal scores): T = the largest
// key x with #{keys >= x} >= kk, bit by bit over the order-preserving keys,
// then one ballot pass in block order.  each_score(f) calls f(j, score of
// block lane + 64 j) for the row's slots in order, -inf past its candidates.
template <typename EachScore>
__device__ __forceinline__ void select_by_bits(EachScore&& each_score, int kk, int32_t* dst, int lane) {
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

// PER > 0: a row's candidates (at most 64 * PER) are loaded once into
// registers, the next row's while the current one is selected; PER == 0 (rows
// beyond 8192 blocks; k_block_topk_wg takes those of 2049 .. 8192): each of
// the two passes over the row streams it, eight loads in flight.
// Waves per SIMD the register budget is fitted to: eight (64 VGPRs) while the
// row fits 16 slots, four beyond (the 32-slot rows' two register sets).  The
// kernel waits mostly on its loads, and eight waves keep twice the rows in
// flight of the five or six the unconstrained allocation leaves room for.
template <int PER>
constexpr int topk_waves() { return PER > 16 ? 4 : 8; }

template <int PER, bool VL, bool K16>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(topk_waves<PER>(), 8))) void k_block_topk(
    const float* __restrict__ pooled, int32_t* __restrict__ out, Dims D, int nrows) {
  // scores >= tau ([w][0][i]) and their blocks' bits ([w][1][i]): a slot's
  // scores are written from entry min(total, 64) on, so the list holds the
  // first 64 in order and a row with more (whose list is not used) stays
  // inside it
  __shared__ float cand[4][2][128];
  // the wave index as a uniform value, so that the rows' buffer descriptors
  // live in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int stride = gridDim.x * 4;
  const float NEG_INF = -__builtin_huge_valf();
  const int k = D.k, kk = k - 1;  // kk blocks to pick among a row's `local` candidates (K16: kk <= 16)
  constexpr int NREG = PER > 0 ? PER : 1;

  // A row (r < nrows: the launch's rows number below 2^31): its local block
  // (-1: nothing to do) and the descriptor of its candidate scores (offsets
  // past the candidates read 0 and never leave them).
  // Rows carry their query index i = r mod n_q and, varlen, their sequence b
  // and offset rb = r mod (h_kv n_q) inside it; the walk advances them by the
  // stride's quotient and remainder instead of dividing each row.
  struct Row {
    int r, i, b, rb, local;
    __amdgpu_buffer_rsrc_t rs;
  };
  const int per_seq = D.h_kv * D.n_q;  // rows of one sequence
  const int step_i = stride % D.n_q, step_rb = stride % per_seq, step_b = stride / per_seq;
  auto finish = [&](Row& x) {
    x.local = -1;
    if (x.r < nrows) {
      if constexpr (VL) {
        if (x.i < seq_nq(D, x.b)) x.local = (int)((seq_offset(D, x.b) + x.i) / kBk);  // rows past a sequence's queries: none
      } else {
        x.local = (int)((D.offset + x.i) / kBk);
      }
    }
    x.rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(pooled + (int64_t)x.r * D.n_blk), (short)0,
                                             max(x.local, 0) * 4, kRawBufferFlags);
  };
  auto row_at = [&](int r) {
    Row x;
    x.r = r;
    x.i = r % D.n_q;
    x.b = r / per_seq;
    x.rb = r % per_seq;
    finish(x);
    return x;
  };
  auto next_row = [&](const Row& c) {
    Row x;
    x.r = c.r + stride;
    x.i = c.i + step_i;
    if (x.i >= D.n_q) x.i -= D.n_q;
    if constexpr (VL) {
      x.rb = c.rb + step_rb;
      x.b = c.b + step_b;
      if (x.rb >= per_seq) {
        x.rb -= per_seq;
        ++x.b;
      }
    } else {
      x.b = x.rb = 0;
    }
    finish(x);
    return x;
  };
  // `lane` as a value the compiler cannot see through (an empty asm per use
  // site): per-slot values derived from it (offsets, block ids) are then
  // formed where they are used, from one register, instead of being hoisted
  // out of the row loop into one register per slot
  auto opaque_lane = [&]() {
    int v = lane;
    asm volatile("" : "+v"(v));
    return v;
  };
  // slot j's score: the lane's byte offset plus an immediate 256 j
  auto load_at = [&](const Row& x, int off, int j) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(x.rs, off + 256 * j, 0, 0));
  };
  auto load = [&](const Row& x, int j) { return load_at(x, 4 * opaque_lane(), j); };
  // registers of a row's scores: issued now, used later (all PER slots: the
  // ones past the row read 0 through the descriptor and touch no memory)
  auto fetch = [&](const Row& x, float (&v)[NREG]) {
    if constexpr (PER > 0) {
      const int off = 4 * opaque_lane();
#pragma unroll
      for (int j = 0; j < PER; ++j) v[j] = load_at(x, off, j);
    }
  };

  // One row: its block list from its candidate scores (in vc for PER > 0).
  auto select_row = [&](const Row& x, float (&vc)[NREG]) {
    const int local = x.local;
    int32_t* dst = out + (int64_t)x.r * k;
    if (local < 0) return;  // not a row of this batch
    if (local + 1 <= k) {  // every visible block is kept
      for (int s = lane; s < k; s += 64) dst[s] = s <= local ? s : -1;
      return;
    }
    if (kk == 0) {
      if (lane == 0) dst[0] = local;
      return;
    }
    const int nj = (local + 63) >> 6;  // score slots in use (uniform)
    // the registers' scores past the candidates (they read 0) become -inf, in place
    auto mask_tail = [&]() {
      if constexpr (PER > 0) {
        int lim = local;
        asm volatile("" : "+s"(lim));  // keeps the compares on the paths that mask
        const int lv = opaque_lane();
#pragma unroll
        for (int j = 0; j < PER; ++j) vc[j] = lv < lim - 64 * j ? vc[j] : NEG_INF;
      }
    };
    // f(j, score of block lane + 64 j) for j = 0 .. nj-1, in order; only the
    // last slot can reach past the candidates (registers: as they stand)
    auto each_score = [&](auto&& f) {
      if constexpr (PER > 0) {
#pragma unroll
        for (int j = 0; j < PER; ++j)
          if (j < nj) f(j, vc[j]);
      } else {
        for (int j0 = 0; j0 < nj; j0 += 8) {  // eight loads in flight per step
          float v[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) v[u] = load(x, j0 + u);
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (j0 + u < nj) f(j0 + u, lane + 64 * (j0 + u) < local ? v[u] : NEG_INF);
        }
      }
    };
    auto reg_max = [&]() {
      float mx = vc[0];
#pragma unroll
      for (int j = 1; j < NREG; ++j) mx = fmaxf(mx, vc[j]);
      return mx;
    };

    // 1. tau from the lane maxima (rows in registers with kk <= 16: the
    // 16-lane rule; streamed rows keep the tighter 64-lane one: fewer
    // candidates)
    auto tau_of = [&](float mx) { return PER > 0 && K16 ? tau16(mx, kk, lane) : tau64(mx, kk, lane); };
    float tau;
    if constexpr (PER > 0) {
      // First from the registers as loaded, the offsets past the candidates
      // reading 0.  If tau > 0, each lane maximum >= tau is a candidate's
      // score (so at least kk candidates reach tau) and no 0 passes `>= tau`:
      // the row needs no masking.  Otherwise mask and take tau again.
      tau = tau_of(reg_max());
      if (!(tau > 0.0f)) {
        mask_tail();
        tau = tau_of(reg_max());
      }
    } else {
      float mx = NEG_INF;
      each_score([&](int, float c) { mx = fmaxf(mx, c); });
      tau = tau_of(mx);
    }

    // 2. scores >= tau, compacted in ascending block order
    int total = 0;
    const int lane_v = opaque_lane();
    each_score([&](int j, float c) {
      const bool take = c >= tau;
      const uint64_t m = __ballot(take);
      float* at = &cand[wave][0][min(total, 64)];  // uniform
      if (take) {
        const int p = prefix(m);
        at[p] = c;
        at[128 + p] = __int_as_float(lane_v + 64 * j);
      }
      total += __popcll(m);
    });
    if (total <= 64) {
      wave_lds_sync();
      const bool have = lane < total;
      emit_from_list<K16>(have ? cand[wave][0][lane] : NEG_INF, have, __float_as_int(cand[wave][1][lane]), total,
                          kk, dst, lane);
    } else {
      mask_tail();
      select_by_bits(each_score, kk, dst, lane);
    }
    if (lane == 0) dst[kk] = local;
    wave_lds_sync();  // the list is read before the next row overwrites it
  };

  // rows stride apart; with registers, two sets take turns (one selected
  // while the other loads), so that no copy moves the next row's scores
  Row cur = row_at(blockIdx.x * 4 + wave);
  float va[NREG], vb[NREG];
  if constexpr (PER > 0) {
    fetch(cur, va);
    while (cur.r < nrows) {
      Row nxt = next_row(cur);
      fetch(nxt, vb);
      select_row(cur, va);
      cur = nxt;
      if (cur.r >= nrows) break;
      nxt = next_row(cur);
      fetch(nxt, va);
      select_row(cur, vb);
      cur = nxt;
    }
  } else {
    for (; cur.r < nrows; cur = next_row(cur)) select_row(cur, va);
  }
}

// Rows of 2049 .. 8192 blocks: one workgroup of eight waves per row, wave w
// holding blocks 1024 w .. 1024 w + 1023 in registers (block 1024 w + lane +
// 64 j in slot j), so the row is read from memory once (streamed, the second
// pass over a 32 KB row found it evicted and read it again).  The row's tau is
// the kk-th largest of the waves' lane maxima (below).  The waves
// compact their scores >= tau into their own lists (block order within a
// wave, and the waves in block order); wave 0 gathers them and selects as
// above.  A row with more than 64 such scores is selected by wave 0 alone with
// the bitwise search, its scores streamed from memory.
constexpr int kWgWaves = 8, kWgPer = 16, kWgBlocks = kWgWaves * kWgPer * 64;

template <bool VL, bool K16>
__global__ __launch_bounds__(kWgWaves * 64) __attribute__((amdgpu_waves_per_eu(8, 8))) void k_block_topk_wg(
    const float* __restrict__ pooled, int32_t* __restrict__ out, Dims D, int nrows) {
  __shared__ float cand[kWgWaves][2][128];  // per wave, as in k_block_topk
  __shared__ float xtop[2][kWgWaves * 64];  // the waves' largest lane maxima: as loaded, then masked
  __shared__ int xcnt[kWgWaves];            // the waves' counts of scores >= tau
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int stride = gridDim.x;
  const float NEG_INF = -__builtin_huge_valf();
  const int k = D.k, kk = k - 1;
  constexpr int PER = kWgPer;

  struct Row {
    int r, i, b, rb, local, mine;  // mine: this wave's candidates, 0 .. 1024
    __amdgpu_buffer_rsrc_t rs;     // this wave's part of the row
  };
  const int per_seq = D.h_kv * D.n_q;
  const int step_i = stride % D.n_q, step_rb = stride % per_seq, step_b = stride / per_seq;
  auto finish = [&](Row& x) {
    x.local = -1;
    if (x.r < nrows) {
      if constexpr (VL) {
        if (x.i < seq_nq(D, x.b)) x.local = (int)((seq_offset(D, x.b) + x.i) / kBk);
      } else {
        x.local = (int)((D.offset + x.i) / kBk);
      }
    }
    x.mine = min(max(x.local - 1024 * wave, 0), 1024);
    x.rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(pooled + (int64_t)x.r * D.n_blk + 1024 * wave),
                                             (short)0, x.mine * 4, kRawBufferFlags);
  };
  auto row_at = [&](int r) {
    Row x;
    x.r = r;
    x.i = r % D.n_q;
    x.b = r / per_seq;
    x.rb = r % per_seq;
    finish(x);
    return x;
  };
  auto next_row = [&](const Row& c) {
    Row x;
    x.r = c.r + stride;
    x.i = c.i + step_i;
    if (x.i >= D.n_q) x.i -= D.n_q;
    if constexpr (VL) {
      x.rb = c.rb + step_rb;
      x.b = c.b + step_b;
      if (x.rb >= per_seq) {
        x.rb -= per_seq;
        ++x.b;
      }
    } else {
      x.b = x.rb = 0;
    }
    finish(x);
    return x;
  };
  auto opaque_lane = [&]() {
    int v = lane;
    asm volatile("" : "+v"(v));
    return v;
  };
  auto fetch = [&](const Row& x, float (&v)[PER]) {
    const int off = 4 * opaque_lane();
#pragma unroll
    for (int j = 0; j < PER; ++j)
      v[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(x.rs, off + 256 * j, 0, 0));
  };

  auto select_row = [&](const Row& x, float (&vc)[PER]) {
    const int local = x.local, mine = x.mine;  // uniform over the workgroup / the wave
    int32_t* dst = out + (int64_t)x.r * k;
    if (local < 0) return;  // not a row of this batch (the whole workgroup)
    if (local + 1 <= k) {
      if (wave == 0)
        for (int s = lane; s < k; s += 64) dst[s] = s <= local ? s : -1;
      return;
    }
    if (kk == 0) {
      if (wave == 0 && lane == 0) dst[0] = local;
      return;
    }
    const int nj = (mine + 63) >> 6;  // this wave's slots in use
    auto mask_tail = [&]() {
      int lim = __builtin_amdgcn_readfirstlane(mine);
      asm volatile("" : "+s"(lim));
      const int lv = opaque_lane();
#pragma unroll
      for (int j = 0; j < PER; ++j) vc[j] = lv < lim - 64 * j ? vc[j] : NEG_INF;
    };
    auto reg_max = [&]() {
      float mx = vc[0];
#pragma unroll
      for (int j = 1; j < PER; ++j) mx = fmaxf(mx, vc[j]);
      return mx;
    };
    // The row's tau: every wave publishes its kk largest lane maxima (entry
    // w kk + i: wave w's (i+1)-th largest), and each wave folds the 8 kk
    // entries onto its 64 lanes (entry f to lane f mod 64, a maximum) and
    // takes the kk-th largest of those.  Each lane's value is one lane
    // maximum of one wave, a different one per lane, so at least kk lane
    // maxima reach tau; and the largest entries of the row stay apart in the
    // fold, so tau is about the row's kk-th largest lane maximum.
    auto row_tau = [&](int round) {
      const float srt = sort_lanes<64>(reg_max(), lane);  // ascending: lane 63 holds the largest
      if (lane >= 64 - kk) xtop[round][wave * kk + 63 - lane] = srt;
      __syncthreads();
      float x = NEG_INF;
      for (int f = lane; f < kWgWaves * kk; f += 64) x = fmaxf(x, xtop[round][f]);
      return tau64(x, kk, lane);
    };
    // 1. tau, first from the registers as loaded (offsets past a wave's
    // candidates read 0; see k_block_topk), else masked
    float tau = row_tau(0);
    if (!(tau > 0.0f)) {  // uniform over the workgroup
      mask_tail();
      tau = row_tau(1);
    }
    // 2. this wave's scores >= tau into its list
    int total = 0;
    const int lane_v = opaque_lane();
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      if (j < nj) {
        const bool take = vc[j] >= tau;
        const uint64_t m = __ballot(take);
        float* at = &cand[wave][0][min(total, 64)];
        if (take) {
          const int p = prefix(m);
          at[p] = vc[j];
          at[128 + p] = __int_as_float(1024 * wave + lane_v + 64 * j);
        }
        total += __popcll(m);
      }
    }
    if (lane == 0) xcnt[wave] = total;
    __syncthreads();  // every list and count is in LDS
    if (wave == 0) {
      int all = 0, src_off = 0, src = 0;
#pragma unroll
      for (int w = 0; w < kWgWaves; ++w) {
        const int n = xcnt[w];
        if (n > 0 && lane >= all) {  // lane's entry, if any, is in the last nonempty list starting at or before it
          src = w;
          src_off = all;
        }
        all += n;
      }
      if (all <= 64) {
        const bool have = lane < all;
        const int e = have ? lane - src_off : 0;
        emit_from_list<K16>(have ? cand[src][0][e] : NEG_INF, have, __float_as_int(cand[src][1][e]), all, kk, dst,
                            lane);
      } else {
        // the whole row, streamed from memory, -inf past its candidates
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(pooled + (int64_t)x.r * D.n_blk), (short)0, local * 4, kRawBufferFlags);
        const int nj_all = (local + 63) >> 6;
        select_by_bits(
            [&](auto&& f) {  // four loads in flight (the next row's registers are live)
              for (int j0 = 0; j0 < nj_all; j0 += 4) {
                float v[4];
#pragma unroll
                for (int u = 0; u < 4; ++u)
                  v[u] = __builtin_bit_cast(float,
                                            __builtin_amdgcn_raw_buffer_load_b32(rs, 4 * lane + 256 * (j0 + u), 0, 0));
#pragma unroll
                for (int u = 0; u < 4; ++u)
                  if (j0 + u < nj_all) f(j0 + u, lane + 64 * (j0 + u) < local ? v[u] : NEG_INF);
              }
            },
            kk, dst, lane);
      }
      if (lane == 0) dst[kk] = local;
    }
    __syncthreads();  // the lists and counts are read before the next row's
  };

  Row cur = row_at(blockIdx.x);
  float va[PER], vb[PER];
  fetch(cur, va);
  if constexpr (!VL) {
    while (cur.r < nrows) {
      Row nxt = next_row(cur);
      fetch(nxt, vb);
      select_row(cur, va);
      cur = nxt;
      if (cur.r >= nrows) break;
      nxt = next_row(cur);
      fetch(nxt, va);
      select_row(cur, vb);
      cur = nxt;
    }
  } else {
    // varlen rows carry more scalar state: one register set and a copy, which
    // keeps the registers within the eight-wave budget without scratch
    while (cur.r < nrows) {
      const Row nxt = next_row(cur);
      fetch(nxt, vb);
      select_row(cur, va);
      cur = nxt;
#pragma unroll
      for (int j = 0; j < PER; ++j) va[j] = vb[j];
    }
  }
}

}  // namespace

// Workgroups of one kernel resident per CU (at most 8): the grid is that many
// per CU, so that every wave is resident and walks its share of the rows from
// the start.
template <typename Kernel>
int blocks_per_cu(Kernel kernel, int threads) {
  int v = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, reinterpret_cast<const void*>(kernel), threads, 0) !=
          hipSuccess ||
      v <= 0)
    v = 1;
  return std::min(v, 8);
}
template <int P, bool V, bool K>
int topk_blocks_per_cu() {
  static const int nb = blocks_per_cu(&k_block_topk<P, V, K>, 256);
  return nb;
}
template <bool V, bool K>
int topk_wg_blocks_per_cu() {
  static const int nb = blocks_per_cu(&k_block_topk_wg<V, K>, kWgWaves * 64);
  return nb;
}

hipError_t launch_block_topk(const float* pooled, int32_t* block_idx, const Dims& D, hipStream_t stream) {
  const int64_t nrows = (int64_t)D.B * D.h_kv * D.n_q;
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus = n;
  }
  const dim3 block(256);
  const int n = (int)nrows;  // below 2^31 (the problem's row count is checked on the host)
  // scores per lane for the longest row (rows are at most n_blk - 1 candidates)
  const int per = (D.n_blk + 63) / 64;
  auto run = [&](auto per_c, auto vl, auto k16) {
    constexpr int P = decltype(per_c)::value;
    constexpr bool V = decltype(vl)::value, K = decltype(k16)::value;
    const dim3 grid((unsigned)std::min<int64_t>((nrows + 3) / 4, (int64_t)cus * topk_blocks_per_cu<P, V, K>()));
    hipLaunchKernelGGL((k_block_topk<P, V, K>), grid, block, 0, stream, pooled, block_idx, D, n);
    mark("k_block_topk", stream);
  };
  auto go = [&](auto per_c, auto vl) {
    if (decltype(per_c)::value > 0 && D.k - 1 <= 16)
      run(per_c, vl, std::integral_constant<bool, (decltype(per_c)::value > 0)>{});
    else
      run(per_c, vl, std::false_type{});
  };
  // rows of 2049 .. 8192 blocks: a workgroup of eight waves per row
  auto run_wg = [&](auto vl, auto k16) {
    constexpr bool V = decltype(vl)::value, K = decltype(k16)::value;
    const dim3 grid((unsigned)std::min<int64_t>(nrows, (int64_t)cus * topk_wg_blocks_per_cu<V, K>()));
    hipLaunchKernelGGL((k_block_topk_wg<V, K>), grid, dim3(kWgWaves * 64), 0, stream, pooled, block_idx, D, n);
    mark("k_block_topk", stream);
  };
  auto pick = [&](auto vl) {
    if (per <= 4) go(std::integral_constant<int, 4>{}, vl);
    else if (per <= 8) go(std::integral_constant<int, 8>{}, vl);
    else if (per <= 16) go(std::integral_constant<int, 16>{}, vl);
    else if (per <= 32) go(std::integral_constant<int, 32>{}, vl);
    else if (D.n_blk <= kWgBlocks) {
      if (D.k - 1 <= 16) run_wg(vl, std::true_type{});
      else run_wg(vl, std::false_type{});
    } else go(std::integral_constant<int, 0>{}, vl);
  };
  if (dims_varlen(D)) pick(std::true_type{}); else pick(std::false_type{});
  return hipGetLastError();
}

}  // namespace msa
