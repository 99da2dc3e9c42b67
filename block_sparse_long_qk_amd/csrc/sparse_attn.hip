// Main Branch: exact softmax attention over the selected blocks.
//
// Page "MiniMax 发布 MSA 稀疏注意力方法，开源推理内核并推出 MiniMax-M3 模型":
// section 两个分支如何工作 (gather the causally visible tokens of the selected
// blocks; scaled dot-product softmax per query head; the group's heads share
// the block set) and section 内核协同设计 (iterate over KV blocks rather than
// queries, packing gathered query positions into 128x128 score tiles; attention
// and merge run as two separate stages).
//
// Stage A, gather plan (gather_plan.hip): for every (sequence, group, block)
//   the list of query rows that selected it as a non-local block, cut into
//   tiles of `pt` positions (pt * G <= 128 rows for the forward, pt <= 128).
// Stage B, tiles (KV-outer): persistent workgroups of 4 waves claim runs of
//   tiles dynamically (per-XCD counters); the 128-key K block and V block sit
//   in LDS while consecutive tiles stay on one (b, g, block); each wave owns
//   32 of the tile's 128 rows and holds their query vectors in VGPRs, loaded
//   one tile ahead.  S^T = K Q^T and O^T = V^T P^T run on 32x32x16 bf16 MFMA.
//   Non-local tiles need no mask (the block lies wholly before the query);
//   local tiles (pt consecutive positions sharing their local block) apply
//   the causal mask.  Each (row, slot) writes a normalised partial (a 12-bit
//   block-scaled code, see pack_group12) and its base-2 log-sum-exp.
// Stage C, merge: LSE weighting of each row's partials into the bf16 output
//   and the natural-log lse.
//
// Lane layout: a wave owns 32 rows (one MFMA n-tile); lane l holds column
// l % 32, so all softmax statistics of a row live in one lane pair (l, l ^ 32).
#include <algorithm>

#include "fwd_tiles.h"

namespace msa {
namespace {


// Softmax of one wave's raw scores (in place) and the unnormalised
// O^T = V^T P^T.  Returns the row max m2 and sum l in base-2 units
// (score * scale * log2 e).  MASKED drops key key0 + j for rows whose position
// p < key0 + j (local tiles); unmasked tiles see all 128 keys, so the max of
// c * s is c times the max (c >= 0) or the min (c < 0) of the raw scores and
// one fma per score forms the exponent.
template <bool MASKED>
__device__ __forceinline__ void softmax_pv(const uint16_t* Vt, f32x16 (&s)[4], int lane, float c, int64_t key0,
                                           int64_t p, f32x16 (&o)[4], float& m2, float& l) {
  const float NEG_INF = -__builtin_huge_valf();
  const int col = lane & 31, half = lane >> 5;
  if constexpr (MASKED) {
    // key key0 + 32*T + row is visible iff 32*T + row <= p - key0
    const int rel = (int)max<int64_t>(-1, min<int64_t>(kBk, p - key0)) - 4 * half;
    float mx = NEG_INF;
#pragma unroll
    for (int T = 0; T < 4; ++T) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float x = s[T][e] * c;
        if (32 * T + 8 * (e >> 2) + (e & 3) > rel) x = NEG_INF;
        s[T][e] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = fmaxf(mx, wave_xor32(mx));
    const float mref = mx == NEG_INF ? 0.f : mx;  // rows with nothing visible (padding rows)
#pragma unroll
    for (int T = 0; T < 4; ++T) {
#pragma unroll
      for (int e = 0; e < 16; ++e) s[T][e] = __builtin_amdgcn_exp2f(s[T][e] - mref);
    }
    m2 = mx;
  } else {
    float ext;
    if (c >= 0.f) {
      ext = NEG_INF;
#pragma unroll
      for (int T = 0; T < 4; ++T) {
#pragma unroll
        for (int e = 0; e < 16; ++e) ext = fmaxf(ext, s[T][e]);
      }
      ext = fmaxf(ext, wave_xor32(ext));
    } else {
      ext = -NEG_INF;
#pragma unroll
      for (int T = 0; T < 4; ++T) {
#pragma unroll
        for (int e = 0; e < 16; ++e) ext = fminf(ext, s[T][e]);
      }
      ext = fminf(ext, wave_xor32(ext));
    }
    const float mref = ext * c;
#pragma unroll
    for (int T = 0; T < 4; ++T) {
#pragma unroll
      for (int e = 0; e < 16; ++e) s[T][e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[T][e], c, -mref));
    }
    m2 = mref;
  }
  // Masked (local) blocks: each probability enters P V as two bf16 parts,
  // hi = bf16(P) and lo = bf16(P - hi), so the weights carry 16 significant
  // bits instead of 8 (|P - hi - lo| <= 2^-16 P) at the price of a second MFMA
  // per k-step.  A row whose weight sits on a few keys (an early position sees
  // only its local block) needs it: bf16 weights alone could move its output
  // by 2^-8 of its V values.  The local pass is bound by HBM reads, so the
  // extra MFMAs are free there; non-local blocks (128 visible keys each) keep
  // one bf16 pass.
  float sum = 0.f;
#pragma unroll
  for (int T = 0; T < 4; ++T) {
#pragma unroll
    for (int e = 0; e < 16; ++e) sum += s[T][e];
  }
  sum += wave_xor32(sum);
#pragma unroll
  for (int D = 0; D < 4; ++D) o[D] = f32x16{};
  // k-step j = 2T + u covers keys 32T + 16u .. +15.  One pass: its V^T
  // operands are read from LDS while the MFMAs of k-step j-1 run; two passes:
  // right before its eight MFMAs (the other wave of the SIMD covers the read
  // latency, and the registers go to the lo parts)
  const uint16_t* vbase = Vt + col * VP + 4 * half;
  auto read_v = [&](int j, uint4 (&dst)[4]) {
#pragma unroll
    for (int D = 0; D < 4; ++D) {
      const uint16_t* vrow = vbase + 32 * D * VP + 16 * j;
      const uint2 lo = *reinterpret_cast<const uint2*>(vrow);
      const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 8);
      dst[D] = make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
  };
  if constexpr (MASKED) {
    uint4 vf[4];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int T = j >> 1, u = j & 1;
      read_v(j, vf);
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float a = s[T][8 * u + 2 * w], b = s[T][8 * u + 2 * w + 1];
        hi[w] = pack_bf16x2(a, b);
        lo[w] = pack_bf16x2(a - __uint_as_float(hi[w] << 16), b - __uint_as_float(hi[w] & 0xFFFF0000u));
      }
      const uint4 ph = make_uint4(hi[0], hi[1], hi[2], hi[3]);
      const uint4 pl = make_uint4(lo[0], lo[1], lo[2], lo[3]);
#pragma unroll
      for (int D = 0; D < 4; ++D) o[D] = mfma_32x32x16(vf[D], ph, o[D]);
#pragma unroll
      for (int D = 0; D < 4; ++D) o[D] = mfma_32x32x16(vf[D], pl, o[D]);
    }
    // issue order of the LDS reads and MFMAs (the VALU work interleaves freely)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 1);
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 1);
    }
  } else {
    uint4 vf[2][4];
    read_v(0, vf[0]);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int T = j >> 1, u = j & 1;
      if (j + 1 < 8) read_v(j + 1, vf[(j + 1) & 1]);
      const uint4 pb = make_uint4(pack_bf16x2(s[T][8 * u + 0], s[T][8 * u + 1]), pack_bf16x2(s[T][8 * u + 2], s[T][8 * u + 3]),
                                  pack_bf16x2(s[T][8 * u + 4], s[T][8 * u + 5]), pack_bf16x2(s[T][8 * u + 6], s[T][8 * u + 7]));
#pragma unroll
      for (int D = 0; D < 4; ++D) o[D] = mfma_32x32x16(vf[j & 1][D], pb, o[D]);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 1);
#pragma unroll
    for (int j = 0; j < 7; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 1);
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 1);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 1);
  }
  l = sum;
}

// Partials are stored in a 12-bit block-scaled fixed-point code.  The 32
// values a lane holds of one half of the head dim form a group with one
// power-of-two scale: E is the smallest integer with
// max|value| * (1 + 2^-11) < 2^E, each value is stored as the nearest integer
// of value * 2^(11-E), a 12-bit two's complement code that the margin keeps
// within [-2047, 2047], and E as one signed byte.  A value is off by at most
// half a step, 2^(E-12), which is under max|value| / 2047 of its group; bf16
// would be off by up to |value| / 256.  Eight codes fill three dwords, low
// bits first.
//
// One fma forms a code: x * sc + 1.5 * 2^23 lies in [2^23, 2^24), where the
// float spacing is 1, so the sum is rounded to the nearest integer once and
// the code sits in the low 12 mantissa bits.
__device__ __forceinline__ uint32_t code12_bits(float x, float sc) {
  return __float_as_uint(__builtin_fmaf(x, sc, 12582912.f));
}

__device__ __forceinline__ void pack12x8(const uint32_t (&b)[8], uint32_t* d) {
  constexpr uint32_t M = 0xFFFu;
  d[0] = (b[0] & M) | ((b[1] & M) << 12) | (b[2] << 24);
  d[1] = ((b[2] & M) >> 8) | ((b[3] & M) << 4) | ((b[4] & M) << 16) | (b[5] << 28);
  d[2] = ((b[5] & M) >> 4) | ((b[6] & M) << 8) | (b[7] << 20);
}

__device__ __forceinline__ int sext12(uint32_t x, int lsb) { return (int32_t)(x << (20 - lsb)) >> 20; }

__device__ __forceinline__ void unpack12x8(uint32_t d0, uint32_t d1, uint32_t d2, float (&x)[8]) {
  x[0] = (float)sext12(d0, 0);
  x[1] = (float)sext12(d0, 12);
  x[2] = (float)sext12((d0 >> 24) | (d1 << 8), 0);
  x[3] = (float)sext12(d1, 4);
  x[4] = (float)sext12(d1, 16);
  x[5] = (float)sext12((d1 >> 28) | (d2 << 4), 0);
  x[6] = (float)sext12(d2, 8);
  x[7] = (float)sext12(d2, 20);
}

// The code of one group: the 32 accumulators o[0..1][0..15] times inv (the
// normalisation), as 12 dwords in accumulator order into w[0..2]; returns E.
__device__ __forceinline__ int pack_group12(const f32x16 (&o)[2], float inv, uint4* w) {
  float am = 0.f;
#pragma unroll
  for (int d = 0; d < 2; ++d) {
#pragma unroll
    for (int e = 0; e < 16; e += 2) am = fmaxf(am, fmaxf(fabsf(o[d][e]), fabsf(o[d][e + 1])));  // v_max3
  }
  // 0 for an all-zero group; kept within a signed byte, the lower bound only
  // ever reached by values that code to 0
  const int E = min(127, max(-100, __builtin_amdgcn_frexp_expf(am * (inv * 1.00048828125f))));
  const float sc = __builtin_amdgcn_ldexpf(inv, 11 - E);  // exact: inv times a power of two
  uint32_t dw[12];
#pragma unroll
  for (int uu = 0; uu < 4; ++uu) {
    const int d = uu >> 1, e0 = (uu & 1) * 8;
    uint32_t b[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) b[j] = code12_bits(o[d][e0 + j], sc);
    pack12x8(b, dw + 3 * uu);
  }
#pragma unroll
  for (int j = 0; j < 3; ++j) w[j] = make_uint4(dw[4 * j], dw[4 * j + 1], dw[4 * j + 2], dw[4 * j + 3]);
  return E;
}

// Store a wave's packed partials, their scale exponents and log-sum-exps.
// The partial of one (sequence, group, query, slot) is a block of G x 128
// codes (192 bytes per head) laid out chunk-major: 16-byte chunk c (0..11) of
// head h at (c * G + h) * 16 bytes, chunk 6 * half + u holding w[u] of lane
// (column, half), groups (half of the head dim) h = u / 3.  The exponents of a
// lane's two groups sit in one 16-bit word (group h in byte h) at
// (slot * G + head) * 2 + half.  A wave's 32 rows are whole query positions
// (all G heads) whenever G divides 32, so for each u the lanes of one
// position write (or, in the merge, read) consecutive 16-byte chunks straight
// from the MFMA layout, with no transposition.
__device__ __forceinline__ void store_partials(uint32_t* __restrict__ part_o, uint16_t* __restrict__ part_ex,
                                               float* __restrict__ part_lse, const uint4 (&w)[6], uint32_t ex,
                                               float lse, bool valid, int64_t pblk, int hh, int G, int half) {
  if (valid) {
    if (half == 0) part_lse[pblk * G + hh] = lse;
    // read once, by the merge: streamed past the caches
    __builtin_nontemporal_store((uint16_t)ex, part_ex + (pblk * G + hh) * 2 + half);
    uint64_t a = reinterpret_cast<uint64_t>(part_o + (pblk * G * 12 + 6 * half * G + hh) * 4);
    // the six addresses are formed here, one add each, rather than kept live
    // in registers since the partial was packed
    asm volatile("" : "+v"(a));
    const int64_t step = (int64_t)G * 16;  // bytes between consecutive chunks of one head
    typedef __attribute__((address_space(1))) u32x4* gvec;
#pragma unroll
    for (int u = 0; u < 6; ++u)
      __builtin_nontemporal_store(u32x4{w[u].x, w[u].y, w[u].z, w[u].w}, (gvec)(a + u * step));
  }
}

// K/V staging of the forward kernels (kFThreads threads).  K rows are stored
// unpadded and swizzled: row r at r * 256 bytes, its 16-byte chunk c in slot
// c ^ (r % 16), so the 16 lanes that read one chunk of 16 rows hit 16
// different bank groups.  bf16 K arrives by direct global-to-LDS loads (no
// registers): each wave issues 8 of the block's 32 one-KB instructions, one
// per 4 rows, the 16 lanes of a row fetching its chunks in slot order.  FP8 K
// is widened in registers and written to the same slots.  V is written
// transposed (Vt[d][key], pitch VP) as stage_kv writes it.  Keys at or past
// n_valid repeat key n_valid - 1; FULL blocks (all 128 keys cached, as every
// non-local block is) skip that clamp.  The caller waits for vmcnt(0) and then
// for the workgroup barrier before reading the block.
template <bool KV8, bool FULL>
__device__ __forceinline__ void stage_kv_fwd(unsigned char* Ks, uint16_t* Vt, const void* k, const void* v,
                                             int64_t kv0, int n_valid) {
  if constexpr (FULL) n_valid = kBk;
  int tid = threadIdx.x;
  // the per-lane addresses below are formed at each staging, not hoisted out
  // of the tile loop into registers that would stay live all along it
  asm volatile("" : "+v"(tid));
  const int wave = tid >> 6, lane = tid & 63;
  constexpr int VPER = 512 / kFThreads;  // 4-key x 8-dim V units per thread
  if constexpr (!KV8) {
    const unsigned char* kb = static_cast<const unsigned char*>(k) + kv0 * 2;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int g = 8 * wave + u;
      const int row = 4 * g + (lane >> 4);
      const int c = (lane & 15) ^ (row & 15);
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(kb + (int64_t)min(row, n_valid - 1) * 256 + 16 * c),
                                       (__attribute__((address_space(3))) void*)(Ks + 1024 * g), 16, 0, 0);
    }
    const uint16_t* vb = static_cast<const uint16_t*>(v) + kv0;
    uint4 vr[4 * VPER];
#pragma unroll
    for (int u = 0; u < VPER; ++u) {
      const int c = tid + kFThreads * u;
      const int kq = c >> 4, od = c & 15;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        vr[4 * u + q4] = *reinterpret_cast<const uint4*>(vb + min(kq * 4 + q4, n_valid - 1) * kHeadDim + od * 8);
    }
#pragma unroll
    for (int u = 0; u < VPER; ++u) {
      const int c = tid + kFThreads * u;
      const int kq = c >> 4, od = c & 15;
      const uint32_t* w[4] = {reinterpret_cast<const uint32_t*>(&vr[4 * u + 0]), reinterpret_cast<const uint32_t*>(&vr[4 * u + 1]),
                              reinterpret_cast<const uint32_t*>(&vr[4 * u + 2]), reinterpret_cast<const uint32_t*>(&vr[4 * u + 3])};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int sh = (e & 1) * 16;
        const uint32_t v0 = (w[0][e >> 1] >> sh) & 0xFFFFu, v1 = (w[1][e >> 1] >> sh) & 0xFFFFu;
        const uint32_t v2 = (w[2][e >> 1] >> sh) & 0xFFFFu, v3 = (w[3][e >> 1] >> sh) & 0xFFFFu;
        *reinterpret_cast<uint2*>(Vt + (od * 8 + e) * VP + kq * 4) = make_uint2(v0 | (v1 << 16), v2 | (v3 << 16));
      }
    }
  } else {
    constexpr int KPER = 1024 / kFThreads;  // 16-byte pieces (16 codes) per thread
    const unsigned char* kb = static_cast<const unsigned char*>(k) + kv0;
    const unsigned char* vb = static_cast<const unsigned char*>(v) + kv0;
    uint4 kr[KPER];
    uint2 vr[4 * VPER];
#pragma unroll
    for (int u = 0; u < KPER; ++u) {
      const int c = tid + kFThreads * u;
      kr[u] = *reinterpret_cast<const uint4*>(kb + min(c >> 3, n_valid - 1) * kHeadDim + (c & 7) * 16);
    }
#pragma unroll
    for (int u = 0; u < VPER; ++u) {
      const int c = tid + kFThreads * u;
      const int kq = c >> 4, od = c & 15;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        vr[4 * u + q4] = *reinterpret_cast<const uint2*>(vb + min(kq * 4 + q4, n_valid - 1) * kHeadDim + od * 8);
    }
#pragma unroll
    for (int u = 0; u < KPER; ++u) {
      const int c = tid + kFThreads * u;
      const int row = c >> 3, oc = c & 7;
      unsigned char* base = Ks + row * 256;
      *reinterpret_cast<u32x4*>(base + 16 * ((2 * oc) ^ (row & 15))) = e4m3x8_to_bf16(make_uint2(kr[u].x, kr[u].y));
      *reinterpret_cast<u32x4*>(base + 16 * ((2 * oc + 1) ^ (row & 15))) = e4m3x8_to_bf16(make_uint2(kr[u].z, kr[u].w));
    }
#pragma unroll
    for (int u = 0; u < VPER; ++u) {
      const int c = tid + kFThreads * u;
      const int kq = c >> 4, od = c & 15;
      const u32x4 w0 = e4m3x8_to_bf16(vr[4 * u + 0]), w1 = e4m3x8_to_bf16(vr[4 * u + 1]);
      const u32x4 w2 = e4m3x8_to_bf16(vr[4 * u + 2]), w3 = e4m3x8_to_bf16(vr[4 * u + 3]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int sh = (e & 1) * 16;
        const uint32_t v0 = (w0[e >> 1] >> sh) & 0xFFFFu, v1 = (w1[e >> 1] >> sh) & 0xFFFFu;
        const uint32_t v2 = (w2[e >> 1] >> sh) & 0xFFFFu, v3 = (w3[e >> 1] >> sh) & 0xFFFFu;
        *reinterpret_cast<uint2*>(Vt + (od * 8 + e) * VP + kq * 4) = make_uint2(v0 | (v1 << 16), v2 | (v3 << 16));
      }
    }
  }
}

// S^T = K Q^T against query fragments held in registers, K in the swizzled
// layout of stage_kv_fwd: the MFMA sequence of qk_block (same k-order, same
// accumulation), so the scores are bit-identical.
__device__ __forceinline__ void qk_block_q(const unsigned char* Ks, const uint4 (&qf)[8], int lane, f32x16 (&s)[4]) {
  const int col = lane & 31, half = lane >> 5;
  const unsigned char* kbase = Ks + col * 256;  // rows 32 T + col share col's swizzle
  const int sw = col & 15;
  uint4 kf[2][4];
#pragma unroll
  for (int T = 0; T < 4; ++T) kf[0][T] = *reinterpret_cast<const uint4*>(kbase + 32 * T * 256 + 16 * (half ^ sw));
#pragma unroll
  for (int T = 0; T < 4; ++T) s[T] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const int cb = ks & 1, nb = cb ^ 1;
    if (ks + 1 < 8) {
#pragma unroll
      for (int T = 0; T < 4; ++T)
        kf[nb][T] = *reinterpret_cast<const uint4*>(kbase + 32 * T * 256 + 16 * ((2 * (ks + 1) + half) ^ sw));
    }
#pragma unroll
    for (int T = 0; T < 4; ++T) s[T] = mfma_32x32x16(kf[cb][T], qf[ks], s[T]);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
  for (int ks = 0; ks < 7; ++ks) {
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
}

// softmax_pv<false> with the partial packed as it is produced: P is packed
// to bf16 once, then O^T is formed one half of the head dim at a time (32
// accumulator registers instead of 64) and each half is normalised into its
// group of three packed chunks of w (pack_group12), its exponent in byte h
// of ex.  Every accumulator sums the same MFMAs in the same order as
// softmax_pv.
__device__ __forceinline__ void softmax_pv_packed(const uint16_t* Vt, f32x16 (&s)[4], int lane, float c,
                                                  uint4 (&w)[6], uint32_t& ex, float& m2, float& l) {
  const float NEG_INF = -__builtin_huge_valf();
  const int col = lane & 31, half = lane >> 5;
  float ext;
  if (c >= 0.f) {
    ext = NEG_INF;
#pragma unroll
    for (int T = 0; T < 4; ++T) {
#pragma unroll
      for (int e = 0; e < 16; ++e) ext = fmaxf(ext, s[T][e]);
    }
    ext = fmaxf(ext, wave_xor32(ext));
  } else {
    ext = -NEG_INF;
#pragma unroll
    for (int T = 0; T < 4; ++T) {
#pragma unroll
      for (int e = 0; e < 16; ++e) ext = fminf(ext, s[T][e]);
    }
    ext = fminf(ext, wave_xor32(ext));
  }
  const float mref = ext * c;
#pragma unroll
  for (int T = 0; T < 4; ++T) {
#pragma unroll
    for (int e = 0; e < 16; ++e) s[T][e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[T][e], c, -mref));
  }
  m2 = mref;
  float sum = 0.f;
#pragma unroll
  for (int T = 0; T < 4; ++T) {
#pragma unroll
    for (int e = 0; e < 16; ++e) sum += s[T][e];
  }
  sum += wave_xor32(sum);
  l = sum;
  const float inv = 1.f / sum;
  uint4 pb[8];  // k-step j = 2T + u: keys 32T + 16u .. +15
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int T = j >> 1, u = j & 1;
    pb[j] = make_uint4(pack_bf16x2(s[T][8 * u + 0], s[T][8 * u + 1]), pack_bf16x2(s[T][8 * u + 2], s[T][8 * u + 3]),
                       pack_bf16x2(s[T][8 * u + 4], s[T][8 * u + 5]), pack_bf16x2(s[T][8 * u + 6], s[T][8 * u + 7]));
  }
  const uint16_t* vbase = Vt + col * VP + 4 * half;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    auto read_v2 = [&](int j, uint4 (&dst)[2]) {  // V^T rows of dims 32 (2h + d) + col at k-step j
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        const uint16_t* vrow = vbase + 32 * (2 * h + d) * VP + 16 * j;
        const uint2 lo = *reinterpret_cast<const uint2*>(vrow);
        const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 8);
        dst[d] = make_uint4(lo.x, lo.y, hi.x, hi.y);
      }
    };
    f32x16 o[2] = {f32x16{}, f32x16{}};
    uint4 vf[2][2];
    read_v2(0, vf[0]);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j + 1 < 8) read_v2(j + 1, vf[(j + 1) & 1]);
#pragma unroll
      for (int d = 0; d < 2; ++d) o[d] = mfma_32x32x16(vf[j & 1][d], pb[j], o[d]);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int j = 0; j < 7; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    const int E = pack_group12(o, inv, w + 3 * h);
    ex = h == 0 ? (uint32_t)(E & 0xFF) : ex | ((uint32_t)(E & 0xFF) << 8);
  }
}

// a + b, never fused with the product that formed a or b.  The tile step is
// inlined twice (the two query register sets) and a tile runs through either
// copy, so its base-2 lse m2 + log2(l) must not be contracted into an fma in
// one copy and not in the other.
__device__ __forceinline__ float add_exact(float a, float b) {
#pragma clang fp contract(off)
  return a + b;
}

// Runs are handed from thread 0 to the workgroup through three LDS slots: at
// the barrier that starts run r every wave reads run r + 1 from slot
// (r + 1) % 3; thread 0 writes run r + 2 into slot (r + 2) % 3 during run r,
// before the barrier that starts run r + 1.  That slot was last read after
// the barrier that started run r - 1, which every wave has left behind by
// the barrier that started run r, so no wave can still be reading it.

// Non-local tiles (KV-outer, persistent, dynamic runs).  Per tile and wave:
// scores from the query rows in registers; decode of the next tile's list
// entries; stores of the previous tile's partials; the next tile's query rows
// loaded into the other register set; the list entries of the tile after it;
// softmax and P.V, packed into the partial that is stored one tile later.
// The run after next is claimed at the start of each run.
template <bool VL, bool KV8>
__global__ __launch_bounds__(kFThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_attn_tiles(
    const uint16_t* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v, AttnWs ws, Dims D) {
  __shared__ __align__(16) unsigned char Ks[kBk * 256];
  __shared__ __align__(16) uint16_t Vt[kHeadDim * VP];
  __shared__ int2 runs[3];
  const bool leader = threadIdx.x == 0;
  RunQueue rq;
  if (leader) {
    rq.init(ws.ctr, ws.tile_off[ws.n_bins]);
    const int2 a = rq.claim();
    runs[0] = a;
    runs[1] = a.x >= 0 ? rq.claim() : make_int2(-1, -1);
  }
  lds_barrier();
  int2 run = uniform2(runs[0]), nrun = uniform2(runs[1]);
  if (run.x < 0) return;  // uniform over the workgroup
  if (leader && nrun.x >= 0) rq.prefetch();
  int ri = 0;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 31, half = lane >> 5;
  const int r = wave * 32 + col;
  const int ps = r / D.G, hh = r % D.G;
  auto q_ptr = [&](const TileRow& tr) {  // rows that do not exist read row 0 of the group
    const int g = tr.bg % D.h_kv, b = tr.bg / D.h_kv;
    const int i = tr.valid ? tr.i : 0;
    return q + (qrow_of<VL>(D, b, i) * D.h_q + g * D.G + hh) * kHeadDim;
  };
  // The tile after t1, the successor of tile t (-1: none; -2: the first tile
  // of a run not yet known).  A run claimed from another slice can lie
  // anywhere in the tile range, so whether t1 still belongs to t's run is
  // told by t's place in that run, never by comparing tile numbers across runs.
  auto after = [&](int t, int t1) {
    if (t1 < 0) return -1;
    if (t + 1 < run.y) return t1 + 1 < run.y ? t1 + 1 : nrun.x;  // t1 = t + 1, same run
    return t1 + 1 < nrun.y ? t1 + 1 : -2;                       // t1 starts the next run
  };

  int t = run.x;
  TileRow cur = tile_row<false, VL>(tile_raw<false>(ws, D, t, ps), D, ws, t, ps);
  int t1 = t + 1 < run.y ? t + 1 : nrun.x;
  TileRaw raw1 = t1 >= 0 ? tile_raw<false>(ws, D, t1, ps) : TileRaw{-1, 0};
  uint4 qa[8], qb[8];
  load_q(q_ptr(cur), half, qa);
  uint4 pw[6];
  uint32_t pex = 0;
  int64_t ppblk = 0;
  float plse = 0.f;
  bool pvalid = false, have = false;  // have: a packed partial waits in pw (uniform)
  int staged_bg = -1, staged_t = -1;
  bool fresh = true;  // a barrier was passed since the staged block was last read

  auto step = [&](uint4 (&qc)[8], uint4 (&qn)[8]) -> bool {
    if (cur.bg != staged_bg || cur.t != staged_t) {  // uniform
      if (!fresh) lds_barrier();                    // every wave is done with the staged block
      const int sb = cur.bg / D.h_kv;
      const int64_t kv0 = kvoff_of<VL>(D, sb, cur.bg % D.h_kv, cur.t);
      stage_kv_fwd<KV8, true>(Ks, Vt, k, v, kv0, kBk);  // a non-local block lies wholly before the query
      __builtin_amdgcn_s_waitcnt(kWaitVm0);            // this wave's direct K loads have landed
      lds_barrier();
      staged_bg = cur.bg;
      staged_t = cur.t;
    }
    fresh = false;
    // the last tile of a run: the run after next, claimed when this run
    // started, is resolved now (its counter value has long arrived) and
    // handed over at the barrier that starts the next run
    const bool last = t + 1 >= run.y;  // t ends its run (uniform)
    if (leader && last && t1 >= 0) runs[(ri + 2) % 3] = rq.resolve();
    f32x16 s[4];
    __builtin_amdgcn_sched_barrier(0);
    qk_block_q(Ks, qc, lane, s);
    __builtin_amdgcn_sched_barrier(0);
    const bool more = t1 >= 0;  // uniform
    TileRow nxt = cur;
    if (more) nxt = tile_row<false, VL>(raw1, D, ws, t1, ps);
    __builtin_amdgcn_sched_barrier(0);
    if (have) store_partials(ws.part_o, ws.part_ex, ws.part_lse, pw, pex, plse, pvalid, ppblk, hh, D.G, half);
    if (more) load_q(q_ptr(nxt), half, qn);
    int t2 = after(t, t1);
    TileRaw raw2{-1, 0};
    if (t2 >= 0) raw2 = tile_raw<false>(ws, D, t2, ps);
    float m2, l;
    softmax_pv_packed(Vt, s, lane, D.scale_log2, pw, pex, m2, l);
    ppblk = ((int64_t)cur.bg * D.n_q + cur.i) * (D.k + 1) + cur.s;
    plse = add_exact(m2, __log2f(l));
    pvalid = cur.valid;
    have = true;
    if (!more) return false;
    if (last) {  // t1 starts the next run
      lds_barrier();
      fresh = true;
      run = nrun;
      nrun = uniform2(runs[(ri + 2) % 3]);
      ++ri;
      if (leader && nrun.x >= 0) rq.prefetch();
      if (t2 == -2) {  // the next run holds one tile: the one after it starts the run now known
        t2 = nrun.x;
        if (t2 >= 0) raw2 = tile_raw<false>(ws, D, t2, ps);
      }
    }
    t = t1;
    t1 = t2;
    raw1 = raw2;
    cur = nxt;
    return true;
  };
  while (step(qa, qb) && step(qb, qa)) {
  }
  if (have) store_partials(ws.part_o, ws.part_ex, ws.part_lse, pw, pex, plse, pvalid, ppblk, hh, D.G, half);
}

// Local tiles fused with the merge (persistent, dynamic runs).  Per tile and
// wave: the query rows are loaded into registers, the masked local block gives
// the unnormalised O^T, its max and sum, and the row's non-local partials
// (lse -inf: no partial) are folded in two slots at a time.  Normalised, the
// result is written to `out` (bf16) and `lse` (natural log).
template <bool VL, bool KV8>
__global__ __launch_bounds__(kFThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_attn_local_merge(
    const uint16_t* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v, AttnWs ws,
    uint16_t* __restrict__ out, float* __restrict__ lse_out, Dims D) {
  __shared__ __align__(16) unsigned char Ks[kBk * 256];
  __shared__ __align__(16) uint16_t Vt[kHeadDim * VP];
  __shared__ int2 runs[3];
  const float NEG_INF = -__builtin_huge_valf();
  const bool leader = threadIdx.x == 0;
  RunQueue rq;
  if (leader) {
    rq.init(ws.ctr + kXcds, D.B * D.h_kv * local_tiles<VL>(D));
    const int2 a = rq.claim();
    runs[0] = a;
    runs[1] = a.x >= 0 ? rq.claim() : make_int2(-1, -1);
  }
  lds_barrier();
  int2 run = uniform2(runs[0]), nrun = uniform2(runs[1]);
  if (run.x < 0) return;  // uniform over the workgroup
  if (leader && nrun.x >= 0) rq.prefetch();
  int ri = 0;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 31, half = lane >> 5;
  const int r = wave * 32 + col;
  const int ps = r / D.G, hh = r % D.G;
  int staged_bg = -1, staged_t = -1;
  bool fresh = true;
  for (int t = run.x;;) {
    const TileRow cur = tile_row<true, VL>(TileRaw{-1, 0}, D, ws, t, ps);
    const int g = cur.bg % D.h_kv, b = cur.bg / D.h_kv;
    const int64_t qoff = (qrow_of<VL>(D, b, cur.valid ? cur.i : 0) * D.h_q + g * D.G + hh) * kHeadDim;
    uint4 qf[8];
    load_q(q + qoff, half, qf);
    // The row's non-local partials (chunk-major blocks, see store_partials):
    // this lane's 64 values of each are chunks 6 * half .. 6 * half + 5 of its
    // head, in accumulator order, with their two exponents in one word.  Their log-sum-exps are requested before the
    // local block is computed, so the max over all slots is known before the
    // fold, which therefore never rescales; partial loads run one slot ahead of
    // the fold.
    const int64_t prow = ((int64_t)cur.bg * D.n_q + cur.i) * (D.k + 1);
    const float* lse_p = ws.part_lse + prow * D.G + hh;                                   // slot s at s * G
    const uint32_t* o_p = ws.part_o + (prow * D.G * 12 + 6 * half * D.G + hh) * 4;  // slot s at s * G * 48
    const uint16_t* ex_p = ws.part_ex + (prow * D.G + hh) * 2 + half;              // slot s at s * G * 2
    float lv[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float x = lse_p[(int64_t)min(j, D.k - 1) * D.G];
      lv[j] = j < D.k ? x : NEG_INF;
    }
    // slots 0 .. 15 that hold a partial: the local block's slot, the padding
    // and the slots past k-1 hold none, and their values are not read
    uint32_t has = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) has |= (lv[j] != NEG_INF ? 1u : 0u) << j;
    auto load_slot = [&](int s0, float& ls, uint4 (&x)[6], uint32_t& ex) {  // past slot k-1: weight 0
      const int sl = min(s0, D.k - 1);
      ls = s0 < D.k ? lse_p[(int64_t)sl * D.G] : NEG_INF;
      const bool used = s0 < 16 ? ((has >> s0) & 1u) != 0 : ls != NEG_INF;
      const uint32_t* src = o_p + (int64_t)sl * D.G * 48;
      if (used) {
        ex = __builtin_nontemporal_load(ex_p + (int64_t)sl * D.G * 2);
#pragma unroll
        for (int u = 0; u < 6; ++u) {  // read once: streamed past the caches
          const u32x4 y = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + u * D.G * 4));
          x[u] = make_uint4(y.x, y.y, y.z, y.w);
        }
      } else {
        ex = 0;
#pragma unroll
        for (int u = 0; u < 6; ++u) x[u] = make_uint4(0u, 0u, 0u, 0u);
      }
    };

    if (cur.bg != staged_bg || cur.t != staged_t) {  // uniform
      if (!fresh) lds_barrier();
      const int sb = cur.bg / D.h_kv;
      const int64_t kv0 = kvoff_of<VL>(D, sb, cur.bg % D.h_kv, cur.t);
      stage_kv_fwd<KV8, false>(Ks, Vt, k, v, kv0, max(1, min(kBk, nkv_of<VL>(D, sb) - cur.t * kBk)));
      __builtin_amdgcn_s_waitcnt(kWaitVm0);  // this wave's direct K loads have landed
      lds_barrier();
      staged_bg = cur.bg;
      staged_t = cur.t;
    }
    fresh = false;
    f32x16 sc[4], o[4];
    float m2, l;
    float M = NEG_INF;
#pragma unroll
    for (int j = 0; j < 16; ++j) M = fmaxf(M, lv[j]);
    __builtin_amdgcn_sched_barrier(0);
    qk_block_q(Ks, qf, lane, sc);
    __builtin_amdgcn_sched_barrier(0);
    for (int s0 = 16; s0 < D.k; s0 += 8) {  // k > 16
      float lw[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) lw[j] = lse_p[(int64_t)min(s0 + j, D.k - 1) * D.G];
#pragma unroll
      for (int j = 0; j < 8; ++j) M = fmaxf(M, lw[j]);
    }
    softmax_pv<true>(Vt, sc, lane, D.scale_log2, (int64_t)cur.t * kBk, off_of<VL>(D, b) + cur.i, o, m2, l);
    M = fmaxf(M, m2);
    {
      const float rs = __builtin_amdgcn_exp2f(m2 - M);
#pragma unroll
      for (int D4 = 0; D4 < 4; ++D4) {
#pragma unroll
        for (int e = 0; e < 16; ++e) o[D4][e] *= rs;
      }
      l *= rs;
    }
    float L = l;
    auto fold = [&](float ls, const uint4 (&x)[6], uint32_t ex) {  // a slot with no partial holds codes 0
      const float wgt = ls != NEG_INF ? __builtin_amdgcn_exp2f(ls - M) : 0.f;
      L += wgt;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        // group h's values are code * 2^(E - 11): the weight takes the scale
        const int E = (int)(int8_t)(uint8_t)(ex >> (8 * h));
        const float wq = __builtin_amdgcn_ldexpf(wgt, E - 11);
        const uint32_t dw[12] = {x[3 * h].x,     x[3 * h].y,     x[3 * h].z,     x[3 * h].w,
                                 x[3 * h + 1].x, x[3 * h + 1].y, x[3 * h + 1].z, x[3 * h + 1].w,
                                 x[3 * h + 2].x, x[3 * h + 2].y, x[3 * h + 2].z, x[3 * h + 2].w};
#pragma unroll
        for (int uu = 0; uu < 4; ++uu) {
          float c[8];
          unpack12x8(dw[3 * uu], dw[3 * uu + 1], dw[3 * uu + 2], c);
#pragma unroll
          for (int j = 0; j < 8; ++j) o[2 * h + (uu >> 1)][(uu & 1) * 8 + j] += wq * c[j];
        }
      }
    };
    {
      float la, lb;
      uint32_t ea, eb;
      uint4 xa[6], xb[6];
      load_slot(0, la, xa, ea);
      for (int s0 = 0; s0 < D.k; s0 += 2) {
        load_slot(s0 + 1, lb, xb, eb);
        fold(la, xa, ea);
        if (s0 + 1 >= D.k) break;
        load_slot(s0 + 2, la, xa, ea);
        fold(lb, xb, eb);
      }
    }
    if (cur.valid) {
      const float inv = 1.f / L;
      // accumulator (D4, e) of lane (col, half) is head dim 32*D4 + 8*(e/4) + 4*half + e%4
      uint16_t* dst = out + qoff + 4 * half;
#pragma unroll
      for (int D4 = 0; D4 < 4; ++D4) {
#pragma unroll
        for (int a = 0; a < 4; ++a)
          *reinterpret_cast<uint2*>(dst + 32 * D4 + 8 * a) =
              make_uint2(pack_bf16x2(o[D4][4 * a] * inv, o[D4][4 * a + 1] * inv),
                         pack_bf16x2(o[D4][4 * a + 2] * inv, o[D4][4 * a + 3] * inv));
      }
      if (lse_out && half == 0)
        lse_out[((int64_t)b * D.h_q + g * D.G + hh) * D.n_q + cur.i] = (M + __log2f(L)) * 0.69314718055994531f;
    }
    if (t + 1 < run.y) {
      ++t;
      continue;
    }
    if (nrun.x < 0) break;  // uniform
    if (leader) runs[(ri + 2) % 3] = rq.resolve();
    lds_barrier();
    fresh = true;
    run = nrun;
    nrun = uniform2(runs[(ri + 2) % 3]);
    ++ri;
    if (leader && nrun.x >= 0) rq.prefetch();
    t = run.x;
  }
}

}  // namespace

Dims fwd_attn_dims(const Dims& D) {
  Dims F = D;
  int pt = 1;  // pt * G rows fill a tile of kFRows; pt <= Bk keeps a local tile inside one block
  while (pt * 2 * D.G <= kFRows && pt * 2 <= kBk) pt *= 2;
  F.pt = pt;
  return F;
}

namespace {
int fwd_attn_grid() { return 2 * persistent_grid(); }  // two four-wave workgroups per CU
}  // namespace

hipError_t launch_attn_kernels(const uint16_t* q, const void* k, const void* v, uint16_t* out, float* lse,
                               const AttnWs& ws, const Dims& F, hipStream_t stream) {
  auto go = [&](auto vl, auto kv8) {
    constexpr bool VL = decltype(vl)::value, K8 = decltype(kv8)::value;
    hipLaunchKernelGGL((k_attn_tiles<VL, K8>), dim3(fwd_attn_grid()), dim3(kFThreads), 0, stream, q, k, v, ws, F);
    mark("k_attn_tiles", stream);
    hipLaunchKernelGGL((k_attn_local_merge<VL, K8>), dim3(fwd_attn_grid()), dim3(kFThreads), 0, stream, q, k, v, ws,
                       out, lse, F);
    mark("k_attn_local_merge", stream);
  };
  using T = std::true_type;
  using Fa = std::false_type;
  if (dims_varlen(F)) {
    if (F.kv_eb == 1) go(T{}, T{}); else go(T{}, Fa{});
  } else {
    if (F.kv_eb == 1) go(Fa{}, T{}); else go(Fa{}, Fa{});
  }
  return hipGetLastError();
}

hipError_t launch_sparse_attn(const uint16_t* q, const void* k, const void* v, const int32_t* block_idx,
                              uint16_t* out, float* lse, const AttnWs& ws, const Dims& D, hipStream_t stream) {
  const Dims F = fwd_attn_dims(D);
  hipError_t e = launch_gather_plan(block_idx, ws, F, stream);
  if (e != hipSuccess) return e;
  return launch_attn_kernels(q, k, v, out, lse, ws, F, stream);
}

}  // namespace msa
