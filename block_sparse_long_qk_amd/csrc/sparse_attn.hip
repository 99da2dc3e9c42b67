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
//   tiles of `pt` positions (pt * G <= 256 rows, pt <= 128).
// Stage B, tiles (KV-outer): persistent workgroups of 8 waves walk runs of
//   tiles; the 128-key K block and V block sit in LDS while the run stays on
//   one (b, g, block); each wave owns 32 of the tile's 256 rows.  A wave's
//   query rows arrive in its own LDS region by direct global-to-LDS loads
//   issued one tile ahead, and S^T = K Q^T and O^T = V^T P^T run on 32x32x16
//   bf16 MFMA.  Non-local tiles need no mask (the block lies wholly before the
//   query); local tiles (pt consecutive positions sharing their local block)
//   apply the causal mask.  Each (row, slot) writes a normalised bf16 partial
//   and its base-2 log-sum-exp.
// Stage C, merge: LSE weighting of each row's partials into the bf16 output
//   and the natural-log lse.
//
// Lane layout: a wave owns 32 rows (one MFMA n-tile); lane l holds column
// l % 32, so all softmax statistics of a row live in one lane pair (l, l ^ 32).
#include <algorithm>

#include "attn_tiles.h"

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

// The wave's 32 normalised partials, bf16 in lane order: row q's 128 values
// are lane q's 64 then lane q+32's 64, in accumulator order.
__device__ __forceinline__ void pack_partial(const f32x16 (&o)[4], float inv, uint4 (&w)[8]) {
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int Dt = u >> 1, e0 = (u & 1) * 8;
    w[u] = make_uint4(pack_bf16x2(o[Dt][e0 + 0] * inv, o[Dt][e0 + 1] * inv),
                      pack_bf16x2(o[Dt][e0 + 2] * inv, o[Dt][e0 + 3] * inv),
                      pack_bf16x2(o[Dt][e0 + 4] * inv, o[Dt][e0 + 5] * inv),
                      pack_bf16x2(o[Dt][e0 + 6] * inv, o[Dt][e0 + 7] * inv));
  }
}

// Store a wave's packed partials and their log-sum-exps.  The partials of one
// (sequence, group, query, slot) form a block of G x 128 bf16 laid out
// chunk-major: 16-byte chunk c of head h at (c * G + h) * 16 bytes, chunk
// 8 * half + u holding w[u] of lane (column, half).  A wave's 32 rows are
// whole query positions (all G heads) whenever G divides 32, so for each u
// the lanes of one position write (or, in the merge, read) consecutive 16-byte
// chunks straight from the MFMA layout, with no transposition.
__device__ __forceinline__ void store_partials(uint16_t* __restrict__ part_o, float* __restrict__ part_lse,
                                               const uint4 (&w)[8], float lse, bool valid, int64_t pblk, int hh,
                                               int G, int half) {
  if (valid) {
    if (half == 0) part_lse[pblk * G + hh] = lse;
    uint16_t* dst = part_o + pblk * G * kHeadDim + hh * 8;
#pragma unroll
    for (int u = 0; u < 8; ++u)  // read once, by the merge: streamed past the caches
      __builtin_nontemporal_store(u32x4{w[u].x, w[u].y, w[u].z, w[u].w},
                                  reinterpret_cast<u32x4*>(dst + (8 * half + u) * G * 8));
  }
}

// Persistent and XCD-aware tile kernel, launched once over the gathered
// non-local tiles and once (LOCAL) over the masked local tiles.  One
// workgroup of kWaves waves per CU (2 waves per SIMD); workgroup w runs on XCD
// w % kXcds (the hardware deals workgroups round-robin over the XCDs); XCD x
// owns the contiguous x-th slice of the tile list, and its workgroups walk
// that slice in runs of kRun consecutive tiles (same (b, g, block) as a rule),
// run r going to workgroup r % (grid / kXcds).  So the K/V block in LDS is
// reused across a run, and the query rows gathered at any time come from at
// most kXcds query groups.
//
// Per tile and wave: scores from the query rows in LDS; decode of the next
// tile's list entries; stores of the previous tile's partials; the next
// tile's query rows fetched into the (now free) LDS region; softmax and P.V;
// the partial packed for storing one tile later.  One counter (vmcnt) tracks
// vector loads and stores alike, so a wait for loads waits for every store
// issued before them: issued where they are, the stores and the next rows
// have a whole softmax and P.V to land before the next tile waits for them.
template <bool LOCAL, bool VL, bool KV8>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_attn_tiles(
    const uint16_t* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v, AttnWs ws, Dims D) {
  __shared__ __align__(16) uint16_t Ks[kBk * KP];
  __shared__ __align__(16) uint16_t Vt[kHeadDim * VP];
  __shared__ __align__(16) unsigned char Qs[kWaves][kQRegion];  // per wave: its query rows
  int total;
  if constexpr (LOCAL) {
    total = D.B * D.h_kv * local_tiles<VL>(D);
  } else {
    total = ws.tile_off[ws.n_bins];
  }
  const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds, per_xcd = gridDim.x / kXcds;
  const int lo = (int)((int64_t)total * xcd / kXcds), hi = (int)((int64_t)total * (xcd + 1) / kXcds);
  const int stride = per_xcd * kRun;  // >= kRun
  Walk w0{lo + slot * kRun, lo + slot * kRun, min(lo + slot * kRun + kRun, hi)};
  if (w0.tile >= hi) return;  // uniform over the workgroup

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 31, half = lane >> 5;
  const int r = wave * 32 + col;
  const int ps = r / D.G, hh = r % D.G;
  unsigned char* qw = Qs[wave];
  auto q_ptr = [&](const TileRow& tr) {  // rows that do not exist read row 0 of the group
    const int g = tr.bg % D.h_kv, b = tr.bg / D.h_kv;
    const int i = tr.valid ? tr.i : 0;
    return q + (qrow_of<VL>(D, b, i) * D.h_q + g * D.G + hh) * kHeadDim;
  };

  TileRow cur = tile_row<LOCAL, VL>(tile_raw<LOCAL>(ws, D, w0.tile, ps), D, ws, w0.tile, ps);
  fetch_q_rows(qw, q_ptr(cur), lane);
  Walk w1 = walk_next(w0, stride, hi);
  TileRaw raw1 = tile_raw<LOCAL>(ws, D, min(w1.tile, hi - 1), ps);
  uint4 pw[8];
  int64_t ppblk = 0;
  float plse = 0.f;
  bool pvalid = false, have = false;  // have: a packed partial waits in pw (uniform)
  // outer loop: one staged K/V block; inner loop: the tiles that use it
  while (w0.tile < hi) {
    {
      const int sb = cur.bg / D.h_kv;
      const int64_t kv0 = kvoff_of<VL>(D, sb, cur.bg % D.h_kv, cur.t);
      stage_kv_any<KV8>(Ks, Vt, k, v, kv0, max(1, min(kBk, nkv_of<VL>(D, sb) - cur.t * kBk)));
      __syncthreads();
    }
    const int staged_bg = cur.bg, staged_t = cur.t;
    bool same;
    do {
      f32x16 s[4];
      __builtin_amdgcn_s_waitcnt(kWaitVm0);  // this tile's query rows have landed in LDS
      __builtin_amdgcn_sched_barrier(0);
      qk_block(Ks, qw, lane, s);
      __builtin_amdgcn_sched_barrier(0);
      const bool more = w1.tile < hi;
      // past the last tile: a stand-in decode of the last one (loads stay in bounds, results unused)
      const TileRow nxt = tile_row<LOCAL, VL>(raw1, D, ws, min(w1.tile, hi - 1), ps);
      __builtin_amdgcn_sched_barrier(0);
      if (have) store_partials(ws.part_o, ws.part_lse, pw, plse, pvalid, ppblk, hh, D.G, half);
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);  // LDS reads of the region are done before it is refilled
      __builtin_amdgcn_sched_barrier(0);
      fetch_q_rows(qw, q_ptr(nxt), lane);
      Walk w2 = w1;
      if (more) w2 = walk_next(w1, stride, hi);
      const TileRaw raw2 = tile_raw<LOCAL>(ws, D, min(w2.tile, hi - 1), ps);
      f32x16 o[4];
      float m2, l;
      softmax_pv<LOCAL>(Vt, s, lane, D.scale_log2, (int64_t)cur.t * kBk, off_of<VL>(D, cur.bg / D.h_kv) + cur.i, o, m2,
                        l);
      pack_partial(o, 1.f / l, pw);
      ppblk = ((int64_t)cur.bg * D.n_q + cur.i) * (D.k + 1) + cur.s;
      plse = m2 + __log2f(l);
      pvalid = cur.valid;
      have = true;
      w0 = w1;
      w1 = w2;
      raw1 = raw2;
      cur = nxt;
      same = more && cur.bg == staged_bg && cur.t == staged_t;  // uniform
    } while (same);
    __syncthreads();  // every wave is done with the staged block
  }
  if (have) store_partials(ws.part_o, ws.part_lse, pw, plse, pvalid, ppblk, hh, D.G, half);
  __builtin_amdgcn_s_waitcnt(kWaitVm0);  // the last (unused) row fetch has landed before the workgroup ends
}

// Local tiles fused with the merge.  Each workgroup walks the local tiles (pt
// consecutive positions sharing their local block; XCD-aware runs as above).
// Per tile and wave: the query rows arrive by direct loads into the wave's LDS
// region, the masked local block gives the unnormalised O^T, its max and sum
// in registers, and the row's non-local partials (lse -inf: no partial) are
// folded in two slots at a time with a running max.  Normalised, the result is
// written to `out` (bf16) and `lse` (natural log).
template <bool VL, bool KV8>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_attn_local_merge(
    const uint16_t* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v, AttnWs ws,
    uint16_t* __restrict__ out, float* __restrict__ lse_out, Dims D) {
  __shared__ __align__(16) uint16_t Ks[kBk * KP];
  __shared__ __align__(16) uint16_t Vt[kHeadDim * VP];
  __shared__ __align__(16) unsigned char Qs[kWaves][kQRegion];
  const float NEG_INF = -__builtin_huge_valf();
  const int total = D.B * D.h_kv * local_tiles<VL>(D);
  const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds, per_xcd = gridDim.x / kXcds;
  const int lo = (int)((int64_t)total * xcd / kXcds), hi = (int)((int64_t)total * (xcd + 1) / kXcds);
  const int stride = per_xcd * kRun;
  Walk w{lo + slot * kRun, lo + slot * kRun, min(lo + slot * kRun + kRun, hi)};
  if (w.tile >= hi) return;  // uniform over the workgroup

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 31, half = lane >> 5;
  const int r = wave * 32 + col;
  const int ps = r / D.G, hh = r % D.G;
  unsigned char* qw = Qs[wave];
  int staged_bg = -1, staged_t = -1;
  for (; w.tile < hi; w = walk_next(w, stride, hi)) {
    const TileRow cur = tile_row<true, VL>(TileRaw{-1, 0}, D, ws, w.tile, ps);
    const int g = cur.bg % D.h_kv, b = cur.bg / D.h_kv;
    const int64_t qoff = (qrow_of<VL>(D, b, cur.valid ? cur.i : 0) * D.h_q + g * D.G + hh) * kHeadDim;
    fetch_q_rows(qw, q + qoff, lane);
    // The row's non-local partials (chunk-major blocks, see store_partials):
    // this lane's 64 values of each are chunks 8 * half .. 8 * half + 7 of its
    // head, in accumulator order.  Their log-sum-exps are requested before the
    // local block is computed, so the max over all slots is known before the
    // fold, which therefore never rescales; partial loads run one slot ahead of
    // the fold.
    const int64_t prow = ((int64_t)cur.bg * D.n_q + cur.i) * (D.k + 1);
    const float* lse_p = ws.part_lse + prow * D.G + hh;                       // slot s at s * G
    const uint16_t* o_p = ws.part_o + prow * D.G * kHeadDim + (8 * half * D.G + hh) * 8;  // slot s at s * G * 128
    auto load_slot = [&](int s0, float& ls, uint4 (&x)[8]) {  // past slot k-1: weight 0
      const int sl = min(s0, D.k - 1);
      ls = s0 < D.k ? lse_p[(int64_t)sl * D.G] : NEG_INF;
      const uint16_t* src = o_p + (int64_t)sl * D.G * kHeadDim;
#pragma unroll
      for (int u = 0; u < 8; ++u) {  // read once: streamed past the caches
        const u32x4 y = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + u * D.G * 8));
        x[u] = make_uint4(y.x, y.y, y.z, y.w);
      }
    };
    float lv[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float x = lse_p[(int64_t)min(j, D.k - 1) * D.G];
      lv[j] = j < D.k ? x : NEG_INF;
    }

    if (cur.bg != staged_bg || cur.t != staged_t) {  // uniform
      if (staged_bg >= 0) __syncthreads();
      const int sb = cur.bg / D.h_kv;
      const int64_t kv0 = kvoff_of<VL>(D, sb, cur.bg % D.h_kv, cur.t);
      stage_kv_any<KV8>(Ks, Vt, k, v, kv0, max(1, min(kBk, nkv_of<VL>(D, sb) - cur.t * kBk)));
      __syncthreads();
      staged_bg = cur.bg;
      staged_t = cur.t;
    }
    f32x16 sc[4], o[4];
    float m2, l;
    __builtin_amdgcn_s_waitcnt(kWaitVm0);  // the query rows have landed in LDS

    float M = NEG_INF;  // the lse loads were issued after the row fetch: landed too
#pragma unroll
    for (int j = 0; j < 16; ++j) M = fmaxf(M, lv[j]);
    __builtin_amdgcn_sched_barrier(0);
    qk_block(Ks, qw, lane, sc);
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
    auto fold = [&](float ls, const uint4 (&x)[8]) {
      const bool use = ls != NEG_INF;
      const float wgt = use ? __builtin_amdgcn_exp2f(ls - M) : 0.f;
      L += wgt;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t xs[4] = {use ? x[u].x : 0u, use ? x[u].y : 0u, use ? x[u].z : 0u, use ? x[u].w : 0u};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int e = (u & 1) * 8 + 2 * c;
          o[u >> 1][e] += wgt * __uint_as_float(xs[c] << 16);
          o[u >> 1][e + 1] += wgt * __uint_as_float(xs[c] & 0xFFFF0000u);
        }
      }
    };
    {
      float la, lb;
      uint4 xa[8], xb[8];
      load_slot(0, la, xa);
      for (int s0 = 0; s0 < D.k; s0 += 2) {
        load_slot(s0 + 1, lb, xb);
        fold(la, xa);
        if (s0 + 1 >= D.k) break;
        load_slot(s0 + 2, la, xa);
        fold(lb, xb);
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
  }
}

}  // namespace

hipError_t launch_sparse_attn(const uint16_t* q, const void* k, const void* v, const int32_t* block_idx,
                              uint16_t* out, float* lse, const AttnWs& ws, const Dims& D, hipStream_t stream) {
  hipError_t e = launch_gather_plan(block_idx, ws, D, stream);
  if (e != hipSuccess) return e;
  auto go = [&](auto vl, auto kv8) {
    constexpr bool VL = decltype(vl)::value, K8 = decltype(kv8)::value;
    hipLaunchKernelGGL((k_attn_tiles<false, VL, K8>), dim3(persistent_grid()), dim3(kThreads), 0, stream, q, k, v, ws,
                       D);
    mark("k_attn_tiles", stream);
    hipLaunchKernelGGL((k_attn_local_merge<VL, K8>), dim3(persistent_grid()), dim3(kThreads), 0, stream, q, k, v, ws,
                       out, lse, D);
    mark("k_attn_local_merge", stream);
  };
  using T = std::true_type;
  using F = std::false_type;
  if (dims_varlen(D)) {
    if (D.kv_eb == 1) go(T{}, T{}); else go(T{}, F{});
  } else {
    if (D.kv_eb == 1) go(F{}, T{}); else go(F{}, F{});
  }
  return hipGetLastError();
}

}  // namespace msa
