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
//   tiles of `pt` positions (pt * G <= 128 rows).
// Stage B, tiles (KV-outer): persistent workgroups walk runs of tiles; the
//   128-key K block and V block sit in LDS while the run stays on one
//   (b, g, block), the tile's query rows are gathered into registers (the next
//   tile's while the current one computes), and S^T = K Q^T and O^T = V^T P^T
//   run on 32x32x16 bf16 MFMA.  Non-local tiles need no mask (the block lies
//   wholly before the query); local tiles (pt consecutive positions sharing
//   their local block) apply the causal mask.  Each (row, slot) writes a
//   normalised bf16 partial and its base-2 log-sum-exp.
// Stage C, merge: LSE weighting of each row's partials into the bf16 output
//   and the natural-log lse.
//
// Lane layout: a wave owns 32 rows (one MFMA n-tile); lane l holds column
// l % 32, so all softmax statistics of a row live in one lane pair (l, l ^ 32).
#include <algorithm>

#include "launch.h"

namespace msa {
namespace {

constexpr int KP = kHeadDim + 8;   // LDS pitch of K rows (bf16): 16-byte pad
constexpr int kXcds = 8;           // XCDs of an MI355X; workgroups are dealt round-robin over them
constexpr int kRun = 8;            // consecutive tiles one workgroup takes before moving on
constexpr int kMergeBatch = 9;     // partial slots whose loads the merge issues together (k = 8: one batch, 16: two)
constexpr int VP = kBk + 4;        // LDS pitch of V^T rows (bf16): 8-byte pad
constexpr int kPstPitch = 272;     // LDS pitch (bytes) of a partial row being stored: 16-byte pad

// Stage one 128-key block of K (row-major, padded) and V (transposed) into LDS.
// Keys at or past n_valid (n_valid >= 1) repeat key n_valid - 1: finite data
// that the causal mask drops, so the block needs no zero fill.  All sixteen
// loads are issued before the first LDS write.
__device__ __forceinline__ void stage_kv(uint16_t* Ks, uint16_t* Vt, const uint16_t* __restrict__ kb,
                                         const uint16_t* __restrict__ vb, int n_valid) {
  const int tid = threadIdx.x;
  uint4 kr[8], vr[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {  // K: 2048 chunks of 16 B
    const int c = tid + 256 * u;
    const int key = min(c >> 4, n_valid - 1), oc = c & 15;
    kr[u] = *reinterpret_cast<const uint4*>(kb + key * kHeadDim + oc * 8);
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {  // V: 512 units of 4 keys x 8 dims
    const int c = tid + 256 * u;
    const int kq = c >> 4, od = c & 15;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      vr[4 * u + q] = *reinterpret_cast<const uint4*>(vb + min(kq * 4 + q, n_valid - 1) * kHeadDim + od * 8);
  }
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int c = tid + 256 * u;
    *reinterpret_cast<uint4*>(Ks + (c >> 4) * KP + (c & 15) * 8) = kr[u];
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {  // written transposed: Vt[d][key]
    const int c = tid + 256 * u;
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
}

// This lane's half of a query row (its 8 k-steps of 8 dims); rows that do not
// exist read a stand-in row (finite data whose results are never stored).
__device__ __forceinline__ void load_q_row(uint4 (&qb)[8], const uint16_t* __restrict__ qrow, int half) {
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) qb[ks] = *reinterpret_cast<const uint4*>(qrow + 16 * ks + 8 * half);
}

// S^T = K Q^T for one wave: the 128 keys of the staged block (4 row tiles of
// 32) against the wave's 32 query rows, raw dot products.  k-steps outer, so
// the four accumulator chains interleave.
__device__ __forceinline__ void qk_block(const uint16_t* Ks, const uint4 (&qb)[8], int lane, f32x16 (&s)[4]) {
  const int col = lane & 31, half = lane >> 5;
#pragma unroll
  for (int T = 0; T < 4; ++T) s[T] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
    for (int T = 0; T < 4; ++T)
      s[T] = mfma_32x32x16(*reinterpret_cast<const uint4*>(Ks + (32 * T + col) * KP + 8 * half + 16 * ks), qb[ks],
                           s[T]);
  }
}

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
  float sum = 0.f;
#pragma unroll
  for (int T = 0; T < 4; ++T) {
#pragma unroll
    for (int e = 0; e < 16; ++e) sum += s[T][e];
  }
  sum += wave_xor32(sum);
#pragma unroll
  for (int D = 0; D < 4; ++D) o[D] = f32x16{};
#pragma unroll
  for (int T = 0; T < 4; ++T) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint4 pb = make_uint4(pack_bf16x2(s[T][8 * u + 0], s[T][8 * u + 1]), pack_bf16x2(s[T][8 * u + 2], s[T][8 * u + 3]),
                                  pack_bf16x2(s[T][8 * u + 4], s[T][8 * u + 5]), pack_bf16x2(s[T][8 * u + 6], s[T][8 * u + 7]));
#pragma unroll
      for (int D = 0; D < 4; ++D) {
        const uint16_t* vrow = Vt + (32 * D + col) * VP + 32 * T + 16 * u + 4 * half;
        const uint2 lo = *reinterpret_cast<const uint2*>(vrow);
        const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 8);
        o[D] = mfma_32x32x16(make_uint4(lo.x, lo.y, hi.x, hi.y), pb, o[D]);
      }
    }
  }
  l = sum;
}

// One lane's row of a tile.  Non-local tiles come from the tile-major gather
// lists (row = query i, slot s of its block_idx row); local tiles are runs of
// pt consecutive positions that share their local block (slot k).
struct TileRow {   // five ints, no padding bytes (which would keep the struct in memory)
  int bg, t;      // (b * h_kv + g), KV block
  int valid;      // this lane's row exists
  int i, s;       // query row (position offset + i), partial slot (k = the local block)
};

// What a lane loads to describe its row of a non-local tile: its list entry,
// which also carries the tile's bin.  Each lane reads its own entry (lanes past
// pt read entry pt - 1), so the bin arrives per lane and nothing waits for it
// until the tile is decoded, a step later.
struct TileRaw {
  int e, bin;
};

template <bool LOCAL>
__device__ __forceinline__ TileRaw tile_raw(const AttnWs& ws, const Dims& D, int tile, int ps) {
  TileRaw r{-1, 0};
  if constexpr (!LOCAL) {
    const int2 x = ws.list[(int64_t)tile * D.pt + min(ps, D.pt - 1)];
    r.e = x.x;
    r.bin = x.y;
  }
  return r;
}

template <bool LOCAL>
__device__ __forceinline__ TileRow tile_row(const TileRaw& raw, const Dims& D, const AttnWs& ws, int tile, int ps) {
  TileRow tr;
  tr.i = 0;
  tr.s = 0;
  if constexpr (!LOCAL) {
    const int bin = __builtin_amdgcn_readfirstlane(raw.bin);  // equal over the tile
    tr.bg = bin / (ws.n_groups * D.n_blk);
    tr.t = bin % D.n_blk;
    tr.valid = ps < D.pt && raw.e >= 0;
    if (tr.valid) {
      tr.i = raw.e / D.k;
      tr.s = raw.e % D.k;
    }
  } else {
    const int64_t a0 = D.offset / D.pt;
    const int n_loc = (int)((D.offset + D.n_q - 1) / D.pt - a0 + 1);
    tr.bg = tile / n_loc;
    const int64_t p0 = (a0 + tile % n_loc) * D.pt;
    tr.t = (int)(p0 / kBk);
    const int64_t p = p0 + ps;
    tr.valid = ps < D.pt && p >= D.offset && p < D.offset + D.n_q;
    if (tr.valid) {
      tr.i = (int)(p - D.offset);
      tr.s = D.k;
    }
  }
  return tr;
}

// Walk of one workgroup over its tiles: runs of kRun consecutive tiles,
// successive runs `stride` apart, inside [.., hi).
struct Walk {
  int tile, run_start, run_end;
};

__device__ __forceinline__ Walk walk_next(const Walk& w, int stride, int hi) {
  Walk n = w;
  if (w.tile + 1 < w.run_end) {
    n.tile = w.tile + 1;
  } else {
    n.run_start = w.run_start + stride;  // stride >= kRun: strictly increasing
    n.tile = n.run_start < hi ? n.run_start : hi;
    n.run_end = min(n.run_start + kRun, hi);
  }
  return n;
}

__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ int64_t shfl_i64(int64_t x, int src) {
  const uint32_t lo = __shfl((uint32_t)x, src, 64);
  const uint32_t hi = __shfl((uint32_t)((uint64_t)x >> 32), src, 64);
  return (int64_t)(((uint64_t)hi << 32) | lo);
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

// Store packed partials and their log-sum-exps.  Stored straight from the MFMA
// layout, one instruction would scatter 64 pieces of 16 bytes over 32 rows;
// instead the rows go through the wave's LDS buffer eight at a time and 16
// consecutive lanes write each 256-byte row.  The buffer's rows are padded to
// 272 bytes: the eight rows then start on different banks, and neither the
// writes (16 lanes, one 128-byte half row each) nor the reads conflict.
__device__ __forceinline__ void store_partials(uint16_t* __restrict__ part_o, float* __restrict__ part_lse,
                                               unsigned char* stage, const uint4 (&w)[8], float lse, bool valid,
                                               int64_t pidx, int lane) {
  const int col = lane & 31, half = lane >> 5;
  if (valid && half == 0) part_lse[pidx] = lse;
#pragma unroll
  for (int rho = 0; rho < 4; ++rho) {
    if ((col >> 3) == rho) {
      unsigned char* dst = stage + (col & 7) * kPstPitch + half * 128;
#pragma unroll
      for (int u = 0; u < 8; ++u) *reinterpret_cast<uint4*>(dst + 16 * u) = w[u];
    }
    wave_lds_fence();
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int chunk = 64 * j + lane;            // 128 chunks of 16 bytes: 8 rows x 256 bytes
      const int rr = chunk >> 4, c16 = chunk & 15;
      const int owner = 8 * rho + rr;             // lane (column) holding that row
      const int64_t rp = shfl_i64(pidx, owner);
      const bool rv = __shfl((int)valid, owner, 64) != 0;
      const uint4 x = *reinterpret_cast<const uint4*>(stage + rr * kPstPitch + c16 * 16);
      if (rv) *reinterpret_cast<uint4*>(part_o + rp * kHeadDim + c16 * 8) = x;
    }
    wave_lds_fence();
  }
}

// Persistent and XCD-aware tile kernel, launched once over the gathered
// non-local tiles and once (LOCAL) over the masked local tiles.  Workgroup w
// runs on XCD w % kXcds (the hardware deals
// workgroups round-robin over the XCDs); XCD x owns the contiguous x-th slice
// of the tile list, and its workgroups walk that slice in runs of kRun
// consecutive tiles (same (b, g, block) as a rule), run r going to workgroup
// r % (grid / kXcds).  So the K/V block in LDS is reused across a run,
// concurrent workgroups of one XCD share K/V blocks through its L2, and the
// query rows gathered at any time come from at most kXcds query groups.  The
// next tile's query rows are fetched while the current tile computes.  Every
// (row, slot) writes a normalised bf16 partial and its base-2 log-sum-exp.
template <bool LOCAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_attn_tiles(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, AttnWs ws,
    Dims D) {
  __shared__ __align__(16) uint16_t Ks[kBk * KP];
  __shared__ __align__(16) uint16_t Vt[kHeadDim * VP];
  __shared__ __align__(16) unsigned char Pst[4][8 * kPstPitch];  // per wave: 8 partial rows on their way out
  int total;
  if constexpr (LOCAL) {
    const int64_t a0 = D.offset / D.pt;
    total = D.B * D.h_kv * (int)((D.offset + D.n_q - 1) / D.pt - a0 + 1);
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
  auto q_row = [&](const TileRow& tr) {  // rows that do not exist read row 0 of the group
    const int g = tr.bg % D.h_kv, b = tr.bg / D.h_kv;
    const int i = tr.valid ? tr.i : 0;
    return q + (((int64_t)b * D.n_q + i) * D.h_q + g * D.G + hh) * kHeadDim;
  };

  // pipeline: the next tile's query rows load into qb once this tile's
  // scores are done with it; the list entries of the tile after that load a
  // step earlier still
  TileRow cur = tile_row<LOCAL>(tile_raw<LOCAL>(ws, D, w0.tile, ps), D, ws, w0.tile, ps);
  uint4 qb[8];
  load_q_row(qb, q_row(cur), half);
  Walk w1 = walk_next(w0, stride, hi);
  TileRaw raw1 = tile_raw<LOCAL>(ws, D, min(w1.tile, hi - 1), ps);
  // A tile's partials are stored one step late, right after the next tile's
  // scores: one counter tracks vector loads and stores alike, so a wait for a
  // load waits for every store issued before it.  Issued there, the stores have
  // a whole softmax and P.V to drain before the wait for the following tile's
  // query rows; the list entries needed next are consumed before them.
  uint4 pw[8];
  int64_t ppidx = 0;
  float plse = 0.f;
  bool pvalid = false, have = false;  // have: a packed partial waits in pw (uniform)
  // outer loop: one staged K/V block; inner loop: the tiles that use it
  while (w0.tile < hi) {
    {
      const int64_t key0 = (int64_t)cur.t * kBk;
      const int64_t kv0 = ((int64_t)cur.bg * D.n_kv + key0) * kHeadDim;
      stage_kv(Ks, Vt, k + kv0, v + kv0, (int)min((int64_t)kBk, (int64_t)D.n_kv - key0));
      __syncthreads();
    }
    const int staged_bg = cur.bg, staged_t = cur.t;
    bool same;
    do {
      f32x16 s[4];
      qk_block(Ks, qb, lane, s);
      const bool more = w1.tile < hi;
      // past the last tile: a stand-in decode of the last one (loads stay in bounds, results unused)
      const TileRow nxt = tile_row<LOCAL>(raw1, D, ws, min(w1.tile, hi - 1), ps);  // before the stores: see above
      __builtin_amdgcn_sched_barrier(0);
      if (have) store_partials(ws.part_o, ws.part_lse, Pst[wave], pw, plse, pvalid, ppidx, lane);
      __builtin_amdgcn_sched_barrier(0);
      load_q_row(qb, q_row(nxt), half);
      Walk w2 = w1;
      if (more) w2 = walk_next(w1, stride, hi);
      const TileRaw raw2 = tile_raw<LOCAL>(ws, D, min(w2.tile, hi - 1), ps);
      f32x16 o[4];
      float m2, l;
      softmax_pv<LOCAL>(Vt, s, lane, D.scale_log2, (int64_t)cur.t * kBk, D.offset + cur.i, o, m2, l);
      pack_partial(o, 1.f / l, pw);
      ppidx = ((((int64_t)cur.bg * D.n_q + cur.i) * (D.k + 1) + cur.s) * D.G + hh);
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
  if (have) store_partials(ws.part_o, ws.part_lse, Pst[wave], pw, plse, pvalid, ppidx, lane);
}

// LSE merge of every row's partials (its non-local slots and the local slot
// k).  One thread per 8 output values of one (row, head): a row-head's 16
// threads read each slot's 256-byte partial contiguously.  Slots without a
// partial carry a log-sum-exp of -inf (set by the gather plan) and weight 0;
// their partial memory is never written, so it is zeroed after the load rather
// than multiplied.  The loads of a batch of slots are all issued before any use.
__global__ __launch_bounds__(256) void k_attn_merge(AttnWs ws, uint16_t* __restrict__ out, float* __restrict__ lse_out,
                                                    Dims D) {
  const float NEG_INF = -__builtin_huge_valf();
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int u = (int)(gid & 15);
  const int64_t rh = gid >> 4;
  const int h = (int)(rh % D.G);
  const int64_t row = rh / D.G;  // (b * h_kv + g) * n_q + i
  if (row >= (int64_t)D.B * D.h_kv * D.n_q) return;
  const int i = (int)(row % D.n_q);
  const int64_t bg = row / D.n_q;
  const float* lse_p = ws.part_lse + row * (D.k + 1) * D.G + h;   // slot s at s * G
  const uint16_t* o_p = ws.part_o + (row * (D.k + 1) * D.G + h) * kHeadDim + 8 * u;  // slot s at s * G * 128
  const int64_t o_stride = (int64_t)D.G * kHeadDim;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float m = NEG_INF, wsum = 0.f;
  for (int s0 = 0; s0 <= D.k; s0 += kMergeBatch) {
    float ls[kMergeBatch];
    uint4 x[kMergeBatch];
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      const int s = min(s0 + j, D.k);  // past slot k: a repeat of slot k, dropped below
      ls[j] = lse_p[s * D.G];
      x[j] = *reinterpret_cast<const uint4*>(o_p + s * o_stride);
    }
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j)
      if (s0 + j > D.k) ls[j] = NEG_INF;
    float mb = m;
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) mb = fmaxf(mb, ls[j]);
    // nothing seen yet (mb = -inf): keep the zeros; else shift to the new max
    const float rescale = mb == NEG_INF ? 1.f : __builtin_amdgcn_exp2f(m - mb);
    wsum *= rescale;
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] *= rescale;
    m = mb;
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      const bool use = ls[j] != NEG_INF;
      const float w = use ? __builtin_amdgcn_exp2f(ls[j] - m) : 0.f;
      wsum += w;
      const uint32_t xs[4] = {use ? x[j].x : 0u, use ? x[j].y : 0u, use ? x[j].z : 0u, use ? x[j].w : 0u};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        acc[2 * c] += w * __uint_as_float(xs[c] << 16);
        acc[2 * c + 1] += w * __uint_as_float(xs[c] & 0xFFFF0000u);
      }
    }
  }
  const float inv = 1.f / wsum;
  // lane order -> head dims: value n = 8*(u%8) + c of half u/8 sits at
  // d = 32*(n/16) + 8*((n%16)/4) + 4*half + n%4
  const int half = u >> 3, v8 = u & 7;
  const int d0 = 32 * (v8 >> 1) + 16 * (v8 & 1) + 4 * half;
  const int g = (int)(bg % D.h_kv), b = (int)(bg / D.h_kv);
  uint16_t* dst = out + (((int64_t)b * D.n_q + i) * D.h_q + g * D.G + h) * kHeadDim;
  *reinterpret_cast<uint2*>(dst + d0) = make_uint2(pack_bf16x2(acc[0] * inv, acc[1] * inv),
                                                  pack_bf16x2(acc[2] * inv, acc[3] * inv));
  *reinterpret_cast<uint2*>(dst + d0 + 8) = make_uint2(pack_bf16x2(acc[4] * inv, acc[5] * inv),
                                                      pack_bf16x2(acc[6] * inv, acc[7] * inv));
  if (lse_out && u == 0)
    lse_out[((int64_t)b * D.h_q + g * D.G + h) * D.n_q + i] = (m + __log2f(wsum)) * 0.69314718055994531f;
}

int persistent_grid() {  // a multiple of kXcds
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) !=
                                                 hipSuccess || n <= 0)
      n = 256;
    cus = n;
  }
  return (2 * cus + kXcds - 1) / kXcds * kXcds;  // two 68 KB-LDS workgroups fit one CU
}

}  // namespace

hipError_t launch_sparse_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* block_idx,
                              uint16_t* out, float* lse, const AttnWs& ws, const Dims& D, hipStream_t stream) {
  hipError_t e = launch_gather_plan(block_idx, ws, D, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_attn_tiles<false>, dim3(persistent_grid()), dim3(256), 0, stream, q, k, v, ws, D);
  hipLaunchKernelGGL(k_attn_tiles<true>, dim3(persistent_grid()), dim3(256), 0, stream, q, k, v, ws, D);
  const int64_t threads = (int64_t)D.B * D.h_kv * D.n_q * D.G * 16;
  hipLaunchKernelGGL(k_attn_merge, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, ws, out, lse, D);
  return hipGetLastError();
}

}  // namespace msa
