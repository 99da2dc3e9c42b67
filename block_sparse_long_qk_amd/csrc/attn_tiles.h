// Tile machinery shared by the KV-outer kernels over the gather plan (the
// sparse attention and the KL alignment pass): LDS geometry, the query-row
// fetch, the description of a tile's rows and the persistent XCD-aware walk.
#pragma once
#include "launch.h"

namespace msa {
namespace {

constexpr int KP = kHeadDim + 8;   // LDS pitch of K rows (bf16): 16-byte pad
constexpr int kXcds = 8;           // XCDs of an MI355X; workgroups are dealt round-robin over them
constexpr int kRun = 8;            // consecutive tiles one workgroup takes before moving on
constexpr int kWaves = 8;          // waves per tile workgroup (kWaves * 32 = 256 rows per tile)
constexpr int kThreads = 64 * kWaves;
constexpr int kQRegion = 32 * 256; // LDS bytes of one wave's 32 query rows
constexpr int VP = kBk + 4;        // LDS pitch of V^T rows (bf16): 8-byte pad

__device__ __forceinline__ uint64_t shfl_u64(uint64_t x, int src) {
  const uint32_t lo = __shfl((uint32_t)x, src, 64);
  const uint32_t hi = __shfl((uint32_t)(x >> 32), src, 64);
  return ((uint64_t)hi << 32) | lo;
}

// A wave's query rows live in its 8 KB LDS region row-major: row r (0..31) at
// r * 256 bytes, its 16-byte chunk c (dims 8c..8c+7) in slot c ^ (r % 16), so
// that the 16 lanes reading one chunk of 16 rows hit 16 different bank groups.
// The rows are fetched with direct global-to-LDS loads, which place lane l's
// 16 bytes at l * 16 past the instruction's LDS address: instruction u fills
// rows 4u..4u+3, the 16 lanes of a row fetching its 16 chunks (permuted), so
// every load instruction reads whole 256-byte rows.  `mine` is the row this
// lane's column owns (lanes l and l ^ 32 own the same one); rows that do not
// exist point at a stand-in row whose results are never stored.
__device__ __forceinline__ void fetch_q_rows(unsigned char* qw, const uint16_t* mine, int lane) {
  const uint64_t me = reinterpret_cast<uint64_t>(mine);
  uint64_t row[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) row[u] = shfl_u64(me, 4 * u + (lane >> 4));
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int r = 4 * u + (lane >> 4);
    const int c = (lane & 15) ^ (r & 15);
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(row[u] + 16 * c),
                                     (__attribute__((address_space(3))) void*)(qw + 1024 * u), 16, 0, 0);
  }
}

// Stage one 128-key block of K (row-major, padded) and V (transposed) into LDS
// with the workgroup's NT threads.  Keys at or past n_valid (n_valid >= 1)
// repeat key n_valid - 1: finite data that the causal mask drops, so the block
// needs no zero fill.  All loads are issued before the first LDS write.
template <int NT = kThreads>
__device__ __forceinline__ void stage_kv(uint16_t* Ks, uint16_t* Vt, const uint16_t* __restrict__ kb,
                                         const uint16_t* __restrict__ vb, int n_valid) {
  constexpr int KPER = 2048 / NT, VPER = 512 / NT;  // 16-byte K chunks, 4-key V units
  const int tid = threadIdx.x;
  uint4 kr[KPER], vr[4 * VPER];
#pragma unroll
  for (int u = 0; u < KPER; ++u) {
    const int c = tid + NT * u;
    const int key = min(c >> 4, n_valid - 1), oc = c & 15;
    kr[u] = *reinterpret_cast<const uint4*>(kb + key * kHeadDim + oc * 8);
  }
#pragma unroll
  for (int u = 0; u < VPER; ++u) {
    const int c = tid + NT * u;
    const int kq = c >> 4, od = c & 15;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      vr[4 * u + q] = *reinterpret_cast<const uint4*>(vb + min(kq * 4 + q, n_valid - 1) * kHeadDim + od * 8);
  }
#pragma unroll
  for (int u = 0; u < KPER; ++u) {
    const int c = tid + NT * u;
    *reinterpret_cast<uint4*>(Ks + (c >> 4) * KP + (c & 15) * 8) = kr[u];
  }
#pragma unroll
  for (int u = 0; u < VPER; ++u) {  // written transposed: Vt[d][key]
    const int c = tid + NT * u;
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

// stage_kv for FP8 E4M3 K and V (1 byte per element, same row layout): the
// same LDS content, each element widened to bf16 between the load and the
// store.  K: 16-byte pieces (16 dims), two per thread; V: 4 keys x 8 dims per
// thread, written transposed as above.
template <int NT = kThreads>
__device__ __forceinline__ void stage_kv8(uint16_t* Ks, uint16_t* Vt, const unsigned char* __restrict__ kb,
                                          const unsigned char* __restrict__ vb, int n_valid) {
  constexpr int KPER = 1024 / NT, VPER = 512 / NT;
  const int tid = threadIdx.x;
  uint4 kr[KPER];
  uint2 vr[4 * VPER];
#pragma unroll
  for (int u = 0; u < KPER; ++u) {
    const int c = tid + NT * u;
    const int key = min(c >> 3, n_valid - 1), oc = c & 7;
    kr[u] = *reinterpret_cast<const uint4*>(kb + key * kHeadDim + oc * 16);
  }
#pragma unroll
  for (int u = 0; u < VPER; ++u) {
    const int c = tid + NT * u;
    const int kq = c >> 4, od = c & 15;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      vr[4 * u + q] = *reinterpret_cast<const uint2*>(vb + min(kq * 4 + q, n_valid - 1) * kHeadDim + od * 8);
  }
#pragma unroll
  for (int u = 0; u < KPER; ++u) {
    const int c = tid + NT * u;
    uint16_t* dst = Ks + (c >> 3) * KP + (c & 7) * 16;
    *reinterpret_cast<u32x4*>(dst) = e4m3x8_to_bf16(make_uint2(kr[u].x, kr[u].y));
    *reinterpret_cast<u32x4*>(dst + 8) = e4m3x8_to_bf16(make_uint2(kr[u].z, kr[u].w));
  }
#pragma unroll
  for (int u = 0; u < VPER; ++u) {  // written transposed: Vt[d][key]
    const int c = tid + NT * u;
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

// K/V block (keys t Bk .. of kv element offset kv0) staged from bf16 or FP8 caches.
template <bool KV8, int NT = kThreads>
__device__ __forceinline__ void stage_kv_any(uint16_t* Ks, uint16_t* Vt, const void* k, const void* v, int64_t kv0,
                                             int n_valid) {
  if constexpr (KV8)
    stage_kv8<NT>(Ks, Vt, static_cast<const unsigned char*>(k) + kv0, static_cast<const unsigned char*>(v) + kv0,
                  n_valid);
  else
    stage_kv<NT>(Ks, Vt, static_cast<const uint16_t*>(k) + kv0, static_cast<const uint16_t*>(v) + kv0, n_valid);
}

// S^T = K Q^T for one wave: the 128 keys of the staged block (4 row tiles of
// 32) against the wave's 32 query rows (from its LDS region), raw dot
// products.  k-steps outer, so the four accumulator chains interleave; the
// operands of k-step ks+1 are read from LDS while the MFMAs of k-step ks run.
__device__ __forceinline__ void qk_block(const uint16_t* Ks, const unsigned char* qw, int lane, f32x16 (&s)[4]) {
  const int col = lane & 31, half = lane >> 5;
  const uint16_t* kbase = Ks + col * KP + 8 * half;
  const unsigned char* qbase = qw + col * 256;
  const int qsw = col & 15;
  uint4 kf[2][4], qf[2];
#pragma unroll
  for (int T = 0; T < 4; ++T) kf[0][T] = *reinterpret_cast<const uint4*>(kbase + 32 * T * KP);
  qf[0] = *reinterpret_cast<const uint4*>(qbase + 16 * (half ^ qsw));
#pragma unroll
  for (int T = 0; T < 4; ++T) s[T] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const int cb = ks & 1, nb = cb ^ 1;
    if (ks + 1 < 8) {
#pragma unroll
      for (int T = 0; T < 4; ++T) kf[nb][T] = *reinterpret_cast<const uint4*>(kbase + 32 * T * KP + 16 * (ks + 1));
      qf[nb] = *reinterpret_cast<const uint4*>(qbase + 16 * ((2 * (ks + 1) + half) ^ qsw));
    }
#pragma unroll
    for (int T = 0; T < 4; ++T) s[T] = mfma_32x32x16(kf[cb][T], qf[cb], s[T]);
  }
  // issue order: the first operands, then per k-step the next operands ahead
  // of that step's four MFMAs
  __builtin_amdgcn_sched_group_barrier(0x100, 5, 0);
#pragma unroll
  for (int ks = 0; ks < 7; ++ks) {
    __builtin_amdgcn_sched_group_barrier(0x100, 5, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
}

// Local tiles per (sequence, group): runs of pt consecutive positions (aligned
// to pt) covering the sequence's query positions; with variable lengths an upper
// bound, the tiles past a sequence's rows having no valid row.
template <bool VL>
__device__ __forceinline__ int local_tiles(const Dims& D) {
  if (VL && (D.qo_lens || D.kv_lens)) return (D.n_q + D.pt - 1) / D.pt + 1;
  return (int)((D.offset + D.n_q - 1) / D.pt - D.offset / D.pt + 1);
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

template <bool LOCAL, bool VL>
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
    const int n_loc = local_tiles<VL>(D);
    tr.bg = tile / n_loc;
    const int b = tr.bg / D.h_kv;
    const int64_t off_b = off_of<VL>(D, b);
    const int64_t p0 = (off_b / D.pt + tile % n_loc) * D.pt;
    tr.t = (int)min(p0 / kBk, (int64_t)D.n_blk - 1);  // tiles past the sequence's rows stay in bounds
    const int64_t p = p0 + ps;
    tr.valid = ps < D.pt && p >= off_b && p < off_b + nq_of<VL>(D, b);
    if (tr.valid) {
      tr.i = (int)(p - off_b);
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

int persistent_grid() {  // a multiple of kXcds
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) !=
                                                 hipSuccess || n <= 0)
      n = 256;
    cus = n;
  }
  return (cus + kXcds - 1) / kXcds * kXcds;  // one 131 KB-LDS workgroup of 8 waves per CU
}


}  // namespace
}  // namespace msa
