// Main Branch backward: dQ, dK, dV of the sparse attention over the selected
// blocks (the gradient that training needs; page "MiniMax 发布 MSA 稀疏注意力方法，
// 开源推理内核并推出 MiniMax-M3 模型", section MSA 如何训练: the language-model loss
// trains the Main Branch, which attends only over the selected blocks).
//
// Per row (query position i, head h) over its token set T:
//   P_j = exp(scale q . k_j - lse),  D = dO . o,
//   dS_j = P_j (dO . v_j - D),  dq = scale sum_j dS_j k_j,
//   dk_j += scale dS_j q,  dv_j += P_j dO.
//
// KV-outer and owner-computes: one workgroup per (sequence, group, block) owns
// that block's dK and dV and walks every row that attends it - the gathered
// rows of the forward's plan (one bin per query group) and the block's own
// positions (masked) - in chunks of 32 rows.  Wave w owns keys 16w .. 16w+15:
// their K and V fragments stay in registers and their dK^T, dV^T accumulate in
// registers over all chunks, so each block is written once, without atomics.
// Per chunk, on 16x16x32 bf16 MFMA (lane l: column l % 16, k-group l / 16):
//   S = Q K_w^T and dP = dO V_w^T with the rows as M: lane (key n, group c)
//   holds rows {4c..4c+3} and {16+4c..16+4c+3}, which is exactly the k-group c
//   that a 32-row contraction reads, so P and dS serve as B operands as they are;
//   dV^T += dO^T P and dK^T += Q^T dS read dO^T and Q^T from the row-major chunk
//   buffers by transposing loads (ds_read_b64_tr_b16);
//   dQ^T = K^T dS^T needs every wave's dS: it goes through LDS once, and wave w
//   forms head dims 16w .. 16w+15 of the chunk's dQ from the staged K^T.
// dQ leaves as one bf16 partial per (row, slot); a merge adds a row's slots.
#include "attn_tiles.h"

namespace msa {
namespace {

typedef __bf16 bf16x8b __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8b, a), __builtin_bit_cast(bf16x8b, b), c,
                                                 0, 0, 0);
}

constexpr int kBwdWaves = 8;
constexpr int kBwdThreads = 64 * kBwdWaves;
constexpr int kTP = 32 + 4;        // pitch (bf16) of the transposed chunk copies [d][32 rows]
constexpr int kKtP = kBk + 8;      // pitch (bf16) of K^T [d][128 keys]

// D[b][h][i] = dO . O for every (row, head): one wave per 8 (row, head) pairs.
__global__ __launch_bounds__(256) void k_bwd_delta(const uint16_t* __restrict__ out, const uint16_t* __restrict__ dout,
                                                   float* __restrict__ delta, Dims D) {
  const int64_t pair = ((int64_t)blockIdx.x * 256 + threadIdx.x) / 8;  // (b, i, h) in out's order
  const int part = threadIdx.x & 7;                                   // 16 head dims each
  if (pair >= (int64_t)D.B * D.n_q * D.h_q) return;
  const uint16_t* o = out + pair * kHeadDim + part * 16;
  const uint16_t* g = dout + pair * kHeadDim + part * 16;
  float acc = 0.f;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const uint4 a = *reinterpret_cast<const uint4*>(o + 8 * u);
    const uint4 b = *reinterpret_cast<const uint4*>(g + 8 * u);
    const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc += __uint_as_float(aw[w] << 16) * __uint_as_float(bw[w] << 16);
      acc += __uint_as_float(aw[w] & 0xFFFF0000u) * __uint_as_float(bw[w] & 0xFFFF0000u);
    }
  }
  acc += __shfl_xor(acc, 1, 64);
  acc += __shfl_xor(acc, 2, 64);
  acc += __shfl_xor(acc, 4, 64);
  if (part == 0) {
    const int h = (int)(pair % D.h_q);
    const int64_t bi = pair / D.h_q;
    const int i = (int)(bi % D.n_q), b = (int)(bi / D.n_q);
    delta[((int64_t)b * D.h_q + h) * D.n_q + i] = acc;
  }
}

// ---------------------------------------------------------------- the chunk walk
// The rows one workgroup walks for its (sequence, group, block): the plan's bin
// of the block for each query group (its entries are compact: list indices
// base .. base + count - 1), then the block's own positions; 32 rows a chunk,
// flattened row R of a source = entry * G + head.  The walk is pipelined: a
// chunk's row table (query row, slot, head of each of its 32 rows) is written
// to LDS two chunks ahead, from list entries loaded one iteration before, so
// every lane can address the next chunk's rows right after a barrier.  The
// table holds ready offsets (one lane per row computes them once), so the
// lanes that use a row do no index arithmetic of their own.
constexpr int kMaxSrc = 260;  // query groups per (b, g) + 1 (n_kv <= 2M: at most 256 groups)
constexpr int kRing = 4;      // row tables in flight: the chunk computed, the one fetched, the one built

struct WalkTab {
  int nent[kMaxSrc];    // entries (positions) of each source
  int base[kMaxSrc];    // bin: first list index; own positions: the first position
  // per chunk row, for query row i of head h at slot s: {position (-1: no row),
  // lse index within the sequence (g G + h) n_q + i, query row within the
  // sequence i h_q + g G + h, h}; an empty row reads row 0 of head 0
  int4 row[kRing][32];
  int64_t part[kRing][32];  // partial offset ((b h_kv + g) n_q + i)(k + 1) + s) rs_mul + h h_mul
  int n_chunks;
};

__device__ __forceinline__ void walk_setup(WalkTab& W, const AttnWs& ws, const Dims& D, int bg, int t) {
  const int n_src = ws.n_groups + 1;
  if (threadIdx.x == 0) W.n_chunks = 0;
  __syncthreads();
  int mine = 0;
  for (int q = threadIdx.x; q < n_src; q += blockDim.x) {
    int nent, base;
    if (q < ws.n_groups) {
      const int bin = (bg * ws.n_groups + q) * D.n_blk + t;
      nent = ws.cnt[bin];
      base = ws.tile_off[bin] * D.pt;
    } else {
      const int lo = max(t * kBk, (int)D.offset), hi = min((t + 1) * kBk, (int)(D.offset + D.n_q));
      nent = max(0, hi - lo);
      base = lo;
    }
    W.nent[q] = nent;
    W.base[q] = base;
    mine += (nent * D.G + 31) / 32;
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) mine += __shfl_xor(mine, m, 64);
  if ((threadIdx.x & 63) == 0 && mine) atomicAdd(&W.n_chunks, mine);
  __syncthreads();
}

// Row-table builder, run by wave 0 (lane r < 32 owns chunk row r).  The
// cursor (source, first row) is uniform over the wave.
struct Builder {
  int src, r0;
  int x;      // pending: list entry (row * k + slot), loaded for every lane (entry 0 if none)
  int kind;   // pending row: 0 none, 1 plan entry x, 2 own position pos
  int pos;    // pending own position
  int h;      // pending row's head
};

__device__ __forceinline__ void bld_skip(Builder& bd, const WalkTab& W, int G, int n_src) {
  while (bd.src < n_src && bd.r0 >= W.nent[bd.src] * G) {
    ++bd.src;
    bd.r0 = 0;
  }
}

// The list load is unconditional (entry 0 when the row is not a plan row), so
// the pending value is defined on every path and needs no copy until its use.
__device__ __forceinline__ void bld_load(Builder& bd, const WalkTab& W, const AttnWs& ws, int G, int n_src,
                                         int lane) {
  const int R = bd.r0 + (lane & 31);
  const bool live = bd.src < n_src && lane < 32 && R < W.nent[min(bd.src, n_src - 1)] * G;
  const bool plan = live && bd.src < n_src - 1;
  const int base = W.base[min(bd.src, n_src - 1)];
  bd.x = ws.list[plan ? base + R / G : 0].x;
  bd.kind = plan ? 1 : (live ? 2 : 0);
  bd.pos = base + R / G;
  bd.h = R % G;
}

// What a kernel's partial offsets are made of: ((bg n_q + i)(k + 1) + s) rs_mul + h h_mul.
struct PartMul {
  int64_t rs;
  int h;
};

__device__ __forceinline__ void bld_write(const Builder& bd, WalkTab& W, int slot, const Dims& D, int bg,
                                          PartMul pm, int lane) {
  if (lane < 32) {
    const int g = bg % D.h_kv;
    int i = -1, sl = 0;
    if (bd.kind == 2) {
      i = (int)(bd.pos - D.offset);
      sl = D.k;
    }
    if (bd.kind == 1 && bd.x >= 0) {
      i = bd.x / D.k;
      sl = bd.x % D.k;
    }
    int4 e = make_int4(-1, 0, 0, 0);
    int64_t off = 0;
    if (i >= 0) {
      e = make_int4((int)(D.offset + i), (g * D.G + bd.h) * D.n_q + i, i * D.h_q + g * D.G + bd.h, bd.h);
      off = (((int64_t)bg * D.n_q + i) * (D.k + 1) + sl) * pm.rs + (int64_t)bd.h * pm.h;
    }
    W.row[slot][lane] = e;
    W.part[slot][lane] = off;
  }
}

__device__ __forceinline__ void bld_next(Builder& bd, const WalkTab& W, int G, int n_src) {
  bd.r0 += 32;
  bld_skip(bd, W, G, n_src);
}

// Tables of chunks 0 and 1 written, chunk 2's entries pending (wave 0 only).
__device__ __forceinline__ void bld_prologue(Builder& bd, WalkTab& W, const AttnWs& ws, const Dims& D, int bg,
                                             PartMul pm, int lane) {
  const int n_src = ws.n_groups + 1;
  bd.src = 0;
  bd.r0 = 0;
  bld_skip(bd, W, D.G, n_src);
  bld_load(bd, W, ws, D.G, n_src, lane);
  bld_write(bd, W, 0, D, bg, pm, lane);
  bld_next(bd, W, D.G, n_src);
  bld_load(bd, W, ws, D.G, n_src, lane);
  bld_write(bd, W, 1, D, bg, pm, lane);
  bld_next(bd, W, D.G, n_src);
  bld_load(bd, W, ws, D.G, n_src, lane);
}

// One iteration of the builder: chunk c + 2's table from the pending entries,
// then chunk c + 3's entries loaded.
__device__ __forceinline__ void bld_step(Builder& bd, WalkTab& W, const AttnWs& ws, const Dims& D, int bg,
                                         PartMul pm, int c, int lane) {
  const int n_src = ws.n_groups + 1;
  bld_write(bd, W, (c + 2) & (kRing - 1), D, bg, pm, lane);
  bld_next(bd, W, D.G, n_src);
  bld_load(bd, W, ws, D.G, n_src, lane);
}

// Transposed chunk copies [d][row] (pitch kTP) with the 4-row quads of dim d
// XOR-swizzled by (d / 16) % 8: element (d, r) at d kTP + 4 ((r / 4) ^ ((d / 16) % 8)) + r % 4.
// With this swizzle (chosen by a bank model of both access patterns) the
// 2-byte writes of a lane's 8 dims of one row and the 8-byte reads of an MFMA
// operand (quads c and 4 + c of dims 16dt .. 16dt+15) each take the minimum
// number of LDS passes; with (d / 8) % 8 both took twice that.
__device__ __forceinline__ int tp_at(int d, int r) { return d * kTP + 4 * ((r >> 2) ^ ((d >> 4) & 7)) + (r & 3); }

// dims 8p .. 8p+7 of row r (one 16-byte register piece) into a transposed copy
__device__ __forceinline__ void tp_store8(uint16_t* dst, u32x4 v, int p, int r) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    dst[tp_at(8 * p + 2 * j, r)] = (uint16_t)(v[j] & 0xFFFFu);
    dst[tp_at(8 * p + 2 * j + 1, r)] = (uint16_t)(v[j] >> 16);
  }
}

// the MFMA operand of dim d: rows 4c .. 4c+3 and 16+4c .. 16+4c+3
__device__ __forceinline__ u32x4 tp_operand(const uint16_t* src, int d, int c) {
  const int sw = (d >> 4) & 7;
  const uint2 a = *reinterpret_cast<const uint2*>(src + d * kTP + 4 * (c ^ sw));
  const uint2 b = *reinterpret_cast<const uint2*>(src + d * kTP + 4 * ((4 + c) ^ sw));
  return u32x4{a.x, a.y, b.x, b.y};
}

typedef short v4s16 __attribute__((ext_vector_type(4)));

// Rows r0 .. r0+3 at dims dbase + (lane % 16), from a row-major chunk buffer
// (row r at 256 r, its 16-byte chunk c in slot c ^ (r % 16)): lane 4e + j of
// each 16-lane group reads row r0 + e, dims dbase + 4j .. +3, and the
// transposing load hands lane i element i % 4 of lanes i / 4 + 4e.
__device__ __forceinline__ uint2 tr_rows4(const unsigned char* buf, int r0, int dbase, int lane) {
  const int e = (lane & 15) >> 2, j = lane & 3;
  const int row = r0 + e, d = dbase + 4 * j;
  const unsigned char* a = buf + row * 256 + 16 * ((d >> 3) ^ (row & 15)) + 2 * (d & 7);
  const v4s16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s16*)a);
  return __builtin_bit_cast(uint2, r);
}

// The 16x16x32 A operand of dims 16 dt + (lane % 16) whose k-group c = lane / 16
// is rows 4c .. 4c+3 and 16+4c .. 16+4c+3 of the chunk (the rows a lane of S
// and dP holds for its key).
__device__ __forceinline__ u32x4 tr_operand16(const unsigned char* buf, int dt, int lane) {
  const int c = lane >> 4;
  const uint2 a = tr_rows4(buf, 4 * c, 16 * dt, lane), b = tr_rows4(buf, 16 + 4 * c, 16 * dt, lane);
  return u32x4{a.x, a.y, b.x, b.y};
}

template <bool VL>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_bwd_kv(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta, AttnWs ws,
    uint16_t* __restrict__ dq_part, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, Dims D) {
  __shared__ __align__(16) uint16_t Kt[kHeadDim * kKtP];             // K^T of the block
  // chunk rows of Q and dO (swizzled), two chunks' worth: chunk c in buffer c % 2
  __shared__ __align__(16) unsigned char Qs[2][32 * 256], Os[2][32 * 256];
  __shared__ __align__(16) unsigned char Ss[32 * 256];  // the chunk's dS [row][key] (swizzled)
  __shared__ WalkTab W;

  // heaviest first: early blocks are candidates for the most rows
  const int nbg = D.B * D.h_kv;
  const int t = (int)(blockIdx.x / nbg);
  const int bg = (int)(blockIdx.x % nbg);
  const int b = bg / D.h_kv, g = bg % D.h_kv;
  const int G = D.G;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, cgrp = lane >> 4;
  const int nkv = D.n_kv;
  const int n_valid = max(1, min(kBk, nkv - t * kBk));
  const uint16_t* kblk = k + (((int64_t)b * D.h_kv + g) * nkv + (int64_t)t * kBk) * kHeadDim;
  const uint16_t* vblk = v + (((int64_t)b * D.h_kv + g) * nkv + (int64_t)t * kBk) * kHeadDim;

  walk_setup(W, ws, D, bg, t);
  const int nch = W.n_chunks;
  Builder bd;
  const PartMul pm{(int64_t)G * kHeadDim, kHeadDim};  // dq partial of (row, slot, head)
  if (wave == 0) bld_prologue(bd, W, ws, D, bg, pm, lane);

  // K^T of the block into LDS (keys past the cache repeat the last one)
  {
    const int tid = threadIdx.x;
    const int kq = tid >> 4, od = tid & 15;  // keys 4kq .. 4kq+3, dims 8od .. 8od+7
    u32x4 x[4];
#pragma unroll
    for (int qq = 0; qq < 4; ++qq)
      x[qq] = *reinterpret_cast<const u32x4*>(kblk + min(4 * kq + qq, n_valid - 1) * kHeadDim + od * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int sh = (e & 1) * 16;
      const uint32_t v0 = (x[0][e >> 1] >> sh) & 0xFFFFu, v1 = (x[1][e >> 1] >> sh) & 0xFFFFu;
      const uint32_t v2 = (x[2][e >> 1] >> sh) & 0xFFFFu, v3 = (x[3][e >> 1] >> sh) & 0xFFFFu;
      *reinterpret_cast<uint2*>(Kt + (od * 8 + e) * kKtP + kq * 4) = make_uint2(v0 | (v1 << 16), v2 | (v3 << 16));
    }
  }
  // this wave's keys as B operands: key 16w + n, dims 32ks + 8c .. +7
  u32x4 kf[4], vf[4];
  {
    const int key = min(16 * wave + n, n_valid - 1);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      kf[ks] = *reinterpret_cast<const u32x4*>(kblk + key * kHeadDim + 32 * ks + 8 * cgrp);
      vf[ks] = *reinterpret_cast<const u32x4*>(vblk + key * kHeadDim + 32 * ks + 8 * cgrp);
    }
  }
  f32x4 dkT[8], dvT[8];  // [d tile]: lane (key n, group c) holds dims 16dt + 4c + e of key 16w + n
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    dkT[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    dvT[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float c2 = D.scale_log2;
  const int key_abs = t * kBk + 16 * wave + n;  // this lane's key (B-operand column)
  __syncthreads();  // row tables of chunks 0 and 1 are written

  // this sequence's rows of Q, dO and their statistics
  const uint16_t* qb = q + (int64_t)b * D.n_q * D.h_q * kHeadDim;
  const uint16_t* ob = dout + (int64_t)b * D.n_q * D.h_q * kHeadDim;
  const float* lseb = lse + (int64_t)b * D.h_q * D.n_q;
  const float* dlb = delta + (int64_t)b * D.h_q * D.n_q;

  // A chunk's rows travel through registers: lane l of wave w loads 16 bytes
  // of row r = 4w + l / 16, its piece p = (l % 16) ^ (r % 16) (dims 8p .. 8p+7),
  // and stores them at byte 1024 w + 16 l of the row buffer (so row r's piece
  // p sits in slot p ^ (r % 16)); dO^T and Q^T are read from these buffers by
  // transposing loads.
  const int my_r = 4 * wave + (lane >> 4);
  const int my_p = (lane & 15) ^ (my_r & 15);
  u32x4 q_next, o_next;
  auto load_rows = [&](int slot) {
    const int64_t qrow = (int64_t)W.row[slot][my_r].z * kHeadDim + 8 * my_p;
    q_next = *reinterpret_cast<const u32x4*>(qb + qrow);
    o_next = *reinterpret_cast<const u32x4*>(ob + qrow);
  };
  auto store_rows = [&](int buf) {
    *reinterpret_cast<u32x4*>(Qs[buf] + 1024 * wave + 16 * lane) = q_next;
    *reinterpret_cast<u32x4*>(Os[buf] + 1024 * wave + 16 * lane) = o_next;
  };
  // raw lse and delta of the next chunk's rows (row 0's for rows that do not
  // exist), first used in the next iteration
  float lse_raw[8], dl_raw[8];
  auto stats = [&](int slot) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int so = W.row[slot][16 * (u >> 2) + 4 * cgrp + (u & 3)].y;
      lse_raw[u] = lseb[so];
      dl_raw[u] = dlb[so];
    }
  };

  // (also without chunks: the table then holds empty rows, which read row 0,
  // and every path reaches the loop with the fragment loads above complete)
  load_rows(0);
  stats(0);
  store_rows(0);
  for (int c = 0; c < nch; ++c) {
    const int slot = c & (kRing - 1);
    const unsigned char* qs = Qs[c & 1];
    const unsigned char* os = Os[c & 1];
    __syncthreads();  // chunk c's rows are in LDS; chunk c + 1's table is visible
    float lse_c[8], dl_c[8];
    int pos8[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int pos = W.row[slot][16 * (u >> 2) + 4 * cgrp + (u & 3)].x;
      const bool ok = pos >= 0;
      pos8[u] = pos;
      lse_c[u] = ok ? lse_raw[u] * 1.4426950408889634f : __builtin_huge_valf();  // P = 0 for rows that do not exist
      dl_c[u] = ok ? dl_raw[u] : 0.f;
      // formed here, before the next chunk's loads are issued (a later use
      // would make its wait count those loads too)
      asm volatile("" ::"v"(lse_c[u]), "v"(dl_c[u]) : "memory");
    }
    if (wave == 0) bld_step(bd, W, ws, D, bg, pm, c, lane);
    // the next chunk's rows and statistics (past the last chunk the table holds
    // empty rows, which read row 0: in bounds and unused)
    load_rows((c + 1) & (kRing - 1));
    stats((c + 1) & (kRing - 1));
    // S = Q K_w^T and dP = dO V_w^T, rows as M (two 16-row tiles)
    f32x4 sc4[2], dp4[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      sc4[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      dp4[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int r = 16 * mt + n;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int sl = (4 * ks + cgrp) ^ (r & 15);
        const u32x4 qa = *reinterpret_cast<const u32x4*>(qs + r * 256 + 16 * sl);
        const u32x4 oa = *reinterpret_cast<const u32x4*>(os + r * 256 + 16 * sl);
        sc4[mt] = mfma16(qa, kf[ks], sc4[mt]);
        dp4[mt] = mfma16(oa, vf[ks], dp4[mt]);
      }
    }
    // P and dS: accumulator u = 4 mt + e is row 16 mt + 4c + e, key 16w + n
    float Pv[8], dS[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float sv = sc4[u >> 2][u & 3];
      const bool vis = key_abs <= pos8[u] && key_abs < nkv;
      const float p = vis ? __builtin_amdgcn_exp2f(__builtin_fmaf(sv, c2, -lse_c[u])) : 0.f;
      Pv[u] = p;
      dS[u] = p * (dp4[u >> 2][u & 3] - dl_c[u]);
    }
    const u32x4 pb = {pack_bf16x2(Pv[0], Pv[1]), pack_bf16x2(Pv[2], Pv[3]), pack_bf16x2(Pv[4], Pv[5]),
                      pack_bf16x2(Pv[6], Pv[7])};
    const u32x4 sb = {pack_bf16x2(dS[0], dS[1]), pack_bf16x2(dS[2], dS[3]), pack_bf16x2(dS[4], dS[5]),
                      pack_bf16x2(dS[6], dS[7])};
    // the chunk's dS for every wave: element (row, key 16w + n) at row * 256 + slot * 16 + 2 (key % 8)
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int r = 16 * (u >> 2) + 4 * cgrp + (u & 3);
      const int key = 16 * wave + n;
      const int sl = (key >> 3) ^ (r & 15);
      *reinterpret_cast<uint16_t*>(Ss + r * 256 + sl * 16 + 2 * (key & 7)) =
          (uint16_t)((u & 1) ? (sb[u >> 1] >> 16) : (sb[u >> 1] & 0xFFFFu));
    }
    __syncthreads();  // dS is in LDS
    // dV^T += dO^T P, dK^T += Q^T dS: M = head dims (8 tiles), K = the 32 rows
    // (k-group c: rows 4c..4c+3 and 16+4c..16+4c+3), N = this wave's keys
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      dvT[dt] = mfma16(tr_operand16(os, dt, lane), pb, dvT[dt]);
      dkT[dt] = mfma16(tr_operand16(qs, dt, lane), sb, dkT[dt]);
    }
    // dQ^T (dims 16w .. 16w+15 x 32 rows) = K^T dS^T over the block's 128 keys;
    // lane (row 16nt + n, group c) holds dims 16w + 4c .. +3 of that row
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const int r = 16 * nt + n;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const u32x4 ka = *reinterpret_cast<const u32x4*>(Kt + (16 * wave + n) * kKtP + 32 * ks + 8 * cgrp);
        const u32x4 sbv = *reinterpret_cast<const u32x4*>(Ss + r * 256 + 16 * ((4 * ks + cgrp) ^ (r & 15)));
        acc = mfma16(ka, sbv, acc);
      }
      if (W.row[slot][r].x >= 0) {
        const float sc = D.scale;
        uint16_t* dst = dq_part + W.part[slot][r] + 16 * wave + 4 * cgrp;
        *reinterpret_cast<uint2*>(dst) =
            make_uint2(pack_bf16x2(acc[0] * sc, acc[1] * sc), pack_bf16x2(acc[2] * sc, acc[3] * sc));
      }
    }
    // chunk c + 1's rows into the other buffer (last read in chunk c - 1,
    // which every wave left before this chunk's first barrier), read after
    // the next barrier
    store_rows((c + 1) & 1);
  }
  // write this wave's keys: lane (key n, group c) holds dims 16dt + 4c .. +3
  if (key_abs < nkv) {
    const int64_t row = (((int64_t)b * D.h_kv + g) * nkv + key_abs) * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const int d = 16 * dt + 4 * cgrp;
      const float sc = D.scale;
      *reinterpret_cast<uint2*>(dk + row + d) = make_uint2(pack_bf16x2(dkT[dt][0] * sc, dkT[dt][1] * sc),
                                                           pack_bf16x2(dkT[dt][2] * sc, dkT[dt][3] * sc));
      *reinterpret_cast<uint2*>(dv + row + d) =
          make_uint2(pack_bf16x2(dvT[dt][0], dvT[dt][1]), pack_bf16x2(dvT[dt][2], dvT[dt][3]));
    }
  }
}

// dq = the sum of a row's slot partials (its listed non-local blocks and the
// local one): one thread per (row, head, 8 dims).
__global__ __launch_bounds__(256) void k_bwd_dq_merge(const int32_t* __restrict__ block_idx,
                                                      const uint16_t* __restrict__ dq_part, uint16_t* __restrict__ dq,
                                                      Dims D) {
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t per_row = (int64_t)D.G * 16;
  const int64_t row = id / per_row;  // (b, g, i)
  if (row >= (int64_t)D.B * D.h_kv * D.n_q) return;
  const int h = (int)((id % per_row) / 16), part = (int)(id % 16);
  const int i = (int)(row % D.n_q);
  const int64_t bg = row / D.n_q;
  const int g = (int)(bg % D.h_kv), b = (int)(bg / D.h_kv);
  const int local = (int)((D.offset + i) / kBk);
  const int32_t* sel = block_idx + row * D.k;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const uint16_t* src = dq_part + (row * (D.k + 1) * D.G + h) * kHeadDim + 8 * part;  // slot s at s G 128
  auto add = [&](uint4 x) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      acc[2 * u] += __uint_as_float(w[u] << 16);
      acc[2 * u + 1] += __uint_as_float(w[u] & 0xFFFF0000u);
    }
  };
  // the listed non-local slots in order, eight loads in flight at a time, then the local slot
  for (int s0 = 0; s0 < D.k; s0 += 8) {
    uint4 x[8];
    bool use[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      use[u] = s0 + u < D.k && nonlocal_slot(sel, s0 + u, local);
      x[u] = use[u] ? *reinterpret_cast<const uint4*>(src + (int64_t)(s0 + u) * D.G * kHeadDim) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (use[u]) add(x[u]);
  }
  add(*reinterpret_cast<const uint4*>(src + (int64_t)D.k * D.G * kHeadDim));
  uint16_t* dst = dq + (((int64_t)b * D.n_q + i) * D.h_q + g * D.G + h) * kHeadDim + 8 * part;
  *reinterpret_cast<uint4*>(dst) = make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                              pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
}

// ---------------------------------------------------------------- KL backward
// Gradient of the KL alignment term into the index projections' outputs, the
// teacher held fixed (page "MiniMax 发布 MSA…", section MSA 如何训练: gradient
// detach keeps the KL loss off the backbone; only the index projections learn
// from it).  With z_j = iq . ik_j, student s_j = exp(z_j - lse_index) and the
// teacher t_j of the forward pass, a row of weight w (d loss / d kl) gives
//   g_j = w (s_j - t_j),  d_iq = sum_j g_j ik_j,  d_ik_j += g_j iq.
// Same owner-computes walk as k_bwd_kv, one workgroup per (sequence, group,
// block): the teacher needs the group's K (S = Q K_w^T over the G head rows
// of each position, summed over the heads), the student Z = IQ IK_w^T with
// every head row reading its position's index-query row; g enters only
// through the position's first head row (the others carry 0), so the same
// 32-row contractions serve: d_ik^T += IQ^T g and d_iq^T = IK^T g^T.  d_ik
// accumulates per group in fp32 (a reduction over groups follows: the index
// keys are shared), d_iq leaves as one bf16 partial per (row, slot).

template <int DIDX, int G>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_kl_bwd(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ iq,
    const uint16_t* __restrict__ ik, const float* __restrict__ lse, const float* __restrict__ lse_index,
    const float* __restrict__ wrow, AttnWs ws, uint16_t* __restrict__ diq_part, float* __restrict__ dik_group,
    Dims D) {
  constexpr int CPI = DIDX / 8;       // 16-byte pieces of an index row
  constexpr int RPI = 64 / CPI;       // index rows per wave instruction
  constexpr int NI = 32 / RPI;        // waves that carry the chunk's index rows
  constexpr int DT = DIDX / 16;       // 16-dim tiles of the index dim
  constexpr int IKS = DIDX / 32;      // k-steps of Z
  __shared__ __align__(16) uint16_t IKt[DIDX * kKtP];         // index keys of the block, transposed
  __shared__ __align__(16) unsigned char Qs[32 * 256];        // the chunk's query rows (swizzled)
  __shared__ __align__(16) unsigned char IQs[32 * 2 * DIDX];  // each row's index-query row (swizzled)
  __shared__ __align__(16) uint16_t IQt[DIDX * kTP];          // its transpose [d][row]
  __shared__ __align__(16) unsigned char Ss[32 * 256];        // the chunk's g [row][key] (swizzled)
  __shared__ WalkTab W;

  const int nbg = D.B * D.h_kv;
  const int t = (int)(blockIdx.x / nbg);
  const int bg = (int)(blockIdx.x % nbg);
  const int b = bg / D.h_kv, g = bg % D.h_kv;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, cgrp = lane >> 4;
  const int nkv = D.n_kv;
  const int n_valid = max(1, min(kBk, nkv - t * kBk));
  const uint16_t* kblk = k + (((int64_t)b * D.h_kv + g) * nkv + (int64_t)t * kBk) * kHeadDim;
  const uint16_t* ikblk = ik + ((int64_t)b * nkv + (int64_t)t * kBk) * DIDX;

  walk_setup(W, ws, D, bg, t);
  const int nch = W.n_chunks;
  Builder bd;
  const PartMul pm{DIDX, 0};  // d_iq partial of (row, slot)
  if (wave == 0) bld_prologue(bd, W, ws, D, bg, pm, lane);

  // the block's index keys transposed into LDS: task = 4 keys x 8 dims
  for (int task = threadIdx.x; task < 32 * CPI; task += kBwdThreads) {
    const int kq = task / CPI, od = task % CPI;
    u32x4 x[4];
#pragma unroll
    for (int qq = 0; qq < 4; ++qq)
      x[qq] = *reinterpret_cast<const u32x4*>(ikblk + min(4 * kq + qq, n_valid - 1) * DIDX + od * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int sh = (e & 1) * 16;
      const uint32_t v0 = (x[0][e >> 1] >> sh) & 0xFFFFu, v1 = (x[1][e >> 1] >> sh) & 0xFFFFu;
      const uint32_t v2 = (x[2][e >> 1] >> sh) & 0xFFFFu, v3 = (x[3][e >> 1] >> sh) & 0xFFFFu;
      *reinterpret_cast<uint2*>(IKt + (od * 8 + e) * kKtP + kq * 4) = make_uint2(v0 | (v1 << 16), v2 | (v3 << 16));
    }
  }
  // this wave's 16 keys as B operands (K of the group, and the index keys)
  u32x4 kf[4], ikf[IKS];
  {
    const int key = min(16 * wave + n, n_valid - 1);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) kf[ks] = *reinterpret_cast<const u32x4*>(kblk + key * kHeadDim + 32 * ks + 8 * cgrp);
#pragma unroll
    for (int ks = 0; ks < IKS; ++ks) ikf[ks] = *reinterpret_cast<const u32x4*>(ikblk + key * DIDX + 32 * ks + 8 * cgrp);
  }
  f32x4 dikT[DT];  // lane (key n, group c): dims 16dt + 4c + e of key 16w + n
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dikT[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float c2 = D.scale_log2;
  constexpr float kL2e = 1.4426950408889634f;
  const int key_abs = t * kBk + 16 * wave + n;
  const bool has_w = wrow != nullptr;
  const float* wsrc = has_w ? wrow : lse_index;  // read either way; 1 is used without weights
  __syncthreads();  // row tables of chunks 0 and 1 are written

  // this sequence's rows and statistics
  const uint16_t* qb = q + (int64_t)b * D.n_q * D.h_q * kHeadDim;
  const uint16_t* iqb = iq + ((int64_t)b * D.n_q * D.h_kv + g) * DIDX;
  const float* lseb = lse + (int64_t)b * D.h_q * D.n_q;
  const float* lzb = lse_index + (int64_t)bg * D.n_q;
  const float* wb = wsrc + (int64_t)bg * D.n_q;

  // A chunk's rows travel through registers, as in the main-branch backward:
  // lane l of wave w carries 16 bytes of query row 4w + l / 16 and (waves
  // below NI) piece p of index row RPI w + l / CPI, stored at byte 1024 w + 16 l
  // and, element by element, into the index rows' transpose.
  const int my_r = 4 * wave + (lane >> 4);
  const int my_ri = RPI * wave + lane / CPI;
  const int my_pi = (lane % CPI) ^ (my_ri % CPI);
  u32x4 q_next, iq_next;
  auto load_rows = [&](int slot) {
    q_next = *reinterpret_cast<const u32x4*>(qb + (int64_t)W.row[slot][my_r].z * kHeadDim +
                                             8 * ((lane & 15) ^ (my_r & 15)));
    if (wave < NI) {
      const int i = max(W.row[slot][my_ri].x - (int)D.offset, 0);
      iq_next = *reinterpret_cast<const u32x4*>(iqb + (int64_t)i * D.h_kv * DIDX + 8 * my_pi);
    }
  };
  auto store_rows = [&]() {
    *reinterpret_cast<u32x4*>(Qs + 1024 * wave + 16 * lane) = q_next;
    if (wave < NI) *reinterpret_cast<u32x4*>(IQs + 1024 * wave + 16 * lane) = iq_next;
  };
  // raw statistics of the next chunk (row 0's for rows that do not exist):
  // the teacher's lse for each of the lane's 8 rows; the student's
  // normaliser and the row weight for its rows 16 m + 4c (m = 0, 1), the only
  // ones that can be a position's first head (G >= 4)
  float lse_raw[8], lz_raw[2], w_raw[2];
  auto stats = [&](int slot) {
#pragma unroll
    for (int u = 0; u < 8; ++u) lse_raw[u] = lseb[W.row[slot][16 * (u >> 2) + 4 * cgrp + (u & 3)].y];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int i = max(W.row[slot][16 * m + 4 * cgrp].x - (int)D.offset, 0);
      lz_raw[m] = lzb[i];
      w_raw[m] = wb[i];
    }
  };

  // (also without chunks: the table then holds empty rows, which read row 0,
  // and every path reaches the loop with the fragment loads above complete)
  load_rows(0);
  stats(0);
  store_rows();
  for (int c = 0; c < nch; ++c) {
    const int slot = c & (kRing - 1);
    __syncthreads();  // chunk c's rows are in LDS; chunk c + 1's table is visible
    // chunk c's index-row transpose, from the registers that still hold its rows
    if (wave < NI) tp_store8(IQt, iq_next, my_pi, my_ri);
    float lse2[8], lz2[2], wg[2];
    int pos8[8];
    bool first[2];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int pos = W.row[slot][16 * (u >> 2) + 4 * cgrp + (u & 3)].x;
      pos8[u] = pos;
      lse2[u] = pos >= 0 ? lse_raw[u] * kL2e : __builtin_huge_valf();
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int4 e = W.row[slot][16 * m + 4 * cgrp];
      first[m] = e.x >= 0 && e.w == 0;
      lz2[m] = lz_raw[m] * kL2e;
      wg[m] = has_w ? w_raw[m] : 1.f;
      asm volatile("" ::"v"(lz2[m]), "v"(wg[m]) : "memory");  // formed before the next chunk's loads
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) asm volatile("" ::"v"(lse2[u]) : "memory");
    if (wave == 0) bld_step(bd, W, ws, D, bg, pm, c, lane);
    load_rows((c + 1) & (kRing - 1));
    stats((c + 1) & (kRing - 1));
    // S (teacher) and Z (student), rows as M
    f32x4 sc4[2], z4[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      sc4[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      z4[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int r = 16 * mt + n;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const u32x4 qa = *reinterpret_cast<const u32x4*>(Qs + r * 256 + 16 * ((4 * ks + cgrp) ^ (r & 15)));
        sc4[mt] = mfma16(qa, kf[ks], sc4[mt]);
      }
#pragma unroll
      for (int ks = 0; ks < IKS; ++ks) {
        const u32x4 ia =
            *reinterpret_cast<const u32x4*>(IQs + r * 2 * DIDX + 16 * ((4 * ks + cgrp) ^ (r % CPI)));
        z4[mt] = mfma16(ia, ikf[ks], z4[mt]);
      }
    }
    // teacher: the head sum of each position (rows 16mt + 4c + e; the heads of
    // a position sit in this lane's e and, for G >= 8, the lanes l ^ 16 and l ^ 32)
    float tsum[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      float sacc = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int u = 4 * mt + e;
        const bool vis = key_abs <= pos8[u] && key_abs < nkv;
        sacc += vis ? __builtin_amdgcn_exp2f(__builtin_fmaf(sc4[mt][e], c2, -lse2[u])) : 0.f;
      }
      tsum[mt] = sacc;
    }
    if constexpr (G >= 8) {
      tsum[0] += __shfl_xor(tsum[0], 16, 64);
      tsum[1] += __shfl_xor(tsum[1], 16, 64);
    }
    if constexpr (G >= 16) {
      tsum[0] += __shfl_xor(tsum[0], 32, 64);
      tsum[1] += __shfl_xor(tsum[1], 32, 64);
    }
    if constexpr (G == 32) tsum[0] = tsum[1] = tsum[0] + tsum[1];
    // g = w (s - t) on each position's first head row (e = 0 of tile m), 0 elsewhere
    float gv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) gv[u] = 0.f;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int u = 4 * m;
      const bool vis = key_abs <= pos8[u] && key_abs < nkv;
      const float sv = vis ? __builtin_amdgcn_exp2f(__builtin_fmaf(z4[m][0], kL2e, -lz2[m])) : 0.f;
      const float tv = vis ? tsum[m] * (1.f / G) : 0.f;
      gv[u] = first[m] ? wg[m] * (sv - tv) : 0.f;
    }
    const u32x4 gb = {pack_bf16x2(gv[0], gv[1]), pack_bf16x2(gv[2], gv[3]), pack_bf16x2(gv[4], gv[5]),
                      pack_bf16x2(gv[6], gv[7])};
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int r = 16 * (u >> 2) + 4 * cgrp + (u & 3);
      const int key = 16 * wave + n;
      const int sl = (key >> 3) ^ (r & 15);
      *reinterpret_cast<uint16_t*>(Ss + r * 256 + sl * 16 + 2 * (key & 7)) =
          (uint16_t)((u & 1) ? (gb[u >> 1] >> 16) : (gb[u >> 1] & 0xFFFFu));
    }
    __syncthreads();  // IQ^T and g are in LDS; the row buffers are free
    // d_ik^T += IQ^T g (M = index dims, K = the 32 rows, N = this wave's keys)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) dikT[dt] = mfma16(tp_operand(IQt, 16 * dt + n, cgrp), gb, dikT[dt]);
    // d_iq^T (dims 16w .. 16w+15 x 32 rows) = IK^T g^T over the block's keys
    if (wave < DT) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        const int r = 16 * nt + n;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const u32x4 ka = *reinterpret_cast<const u32x4*>(IKt + (16 * wave + n) * kKtP + 32 * ks + 8 * cgrp);
          const u32x4 gbv = *reinterpret_cast<const u32x4*>(Ss + r * 256 + 16 * ((4 * ks + cgrp) ^ (r & 15)));
          acc = mfma16(ka, gbv, acc);
        }
        const int4 e = W.row[slot][r];
        if (e.x >= 0 && e.w == 0) {
          uint16_t* dst = diq_part + W.part[slot][r] + 16 * wave + 4 * cgrp;
          *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
        }
      }
    }
    store_rows();  // chunk c + 1's rows, read after the next barrier
  }
  // this group's share of d_ik for the wave's keys (fp32; the groups are added next)
  if (key_abs < nkv) {
    float* dst = dik_group + (((int64_t)b * D.h_kv + g) * nkv + key_abs) * DIDX;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<float4*>(dst + 16 * dt + 4 * cgrp) =
          make_float4(dikT[dt][0], dikT[dt][1], dikT[dt][2], dikT[dt][3]);
  }
}

// The same gradient from a stored teacher (msa_index_kl's optional output:
// fp16 t per (row, slot, key of the block)), so S is not formed again: the
// walk's rows are positions, not head rows (32 positions a chunk), and only
// Z = IQ IK_w^T, g = w (s - t), d_ik^T += IQ^T g and d_iq^T = IK^T g^T remain,
// on the operand layouts of k_kl_bwd.
template <int DIDX>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_kl_bwd_t(
    const uint16_t* __restrict__ iq, const uint16_t* __restrict__ ik, const _Float16* __restrict__ teacher,
    const float* __restrict__ lse_index, const float* __restrict__ wrow, AttnWs ws, uint16_t* __restrict__ diq_part,
    float* __restrict__ dik_group, Dims D) {
  constexpr int CPI = DIDX / 8;       // 16-byte pieces of an index row
  constexpr int RPI = 64 / CPI;       // index rows per wave instruction
  constexpr int NI = 32 / RPI;        // waves that carry the chunk's index rows
  constexpr int DT = DIDX / 16;       // 16-dim tiles of the index dim
  constexpr int IKS = DIDX / 32;      // k-steps of Z
  __shared__ __align__(16) uint16_t IKt[DIDX * kKtP];         // index keys of the block, transposed
  __shared__ __align__(16) unsigned char IQs[32 * 2 * DIDX];  // each row's index-query row (swizzled)
  __shared__ __align__(16) uint16_t IQt[DIDX * kTP];          // its transpose [d][row]
  __shared__ __align__(16) unsigned char Ss[32 * 256];        // the chunk's g [row][key] (swizzled)
  __shared__ WalkTab W;

  Dims D1 = D;  // the walk over positions: one row per plan entry
  D1.G = 1;
  const int nbg = D.B * D.h_kv;
  const int t = (int)(blockIdx.x / nbg);
  const int bg = (int)(blockIdx.x % nbg);
  const int b = bg / D.h_kv, g = bg % D.h_kv;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, cgrp = lane >> 4;
  const int nkv = D.n_kv;
  const int n_valid = max(1, min(kBk, nkv - t * kBk));
  const uint16_t* ikblk = ik + ((int64_t)b * nkv + (int64_t)t * kBk) * DIDX;

  walk_setup(W, ws, D1, bg, t);
  const int nch = W.n_chunks;
  Builder bd;
  const PartMul pm{1, 0};  // the (row, slot) index: d_iq partials DIDX apart, teacher rows kBk apart
  if (wave == 0) bld_prologue(bd, W, ws, D1, bg, pm, lane);

  // the block's index keys transposed into LDS: task = 4 keys x 8 dims
  for (int task = threadIdx.x; task < 32 * CPI; task += kBwdThreads) {
    const int kq = task / CPI, od = task % CPI;
    u32x4 x[4];
#pragma unroll
    for (int qq = 0; qq < 4; ++qq)
      x[qq] = *reinterpret_cast<const u32x4*>(ikblk + min(4 * kq + qq, n_valid - 1) * DIDX + od * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int sh = (e & 1) * 16;
      const uint32_t v0 = (x[0][e >> 1] >> sh) & 0xFFFFu, v1 = (x[1][e >> 1] >> sh) & 0xFFFFu;
      const uint32_t v2 = (x[2][e >> 1] >> sh) & 0xFFFFu, v3 = (x[3][e >> 1] >> sh) & 0xFFFFu;
      *reinterpret_cast<uint2*>(IKt + (od * 8 + e) * kKtP + kq * 4) = make_uint2(v0 | (v1 << 16), v2 | (v3 << 16));
    }
  }
  // this wave's 16 index keys as B operands
  u32x4 ikf[IKS];
  {
    const int key = min(16 * wave + n, n_valid - 1);
#pragma unroll
    for (int ks = 0; ks < IKS; ++ks) ikf[ks] = *reinterpret_cast<const u32x4*>(ikblk + key * DIDX + 32 * ks + 8 * cgrp);
  }
  f32x4 dikT[DT];  // lane (key n, group c): dims 16dt + 4c + e of key 16w + n
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dikT[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  constexpr float kL2e = 1.4426950408889634f;
  const int key_abs = t * kBk + 16 * wave + n;
  const bool has_w = wrow != nullptr;
  const float* wsrc = has_w ? wrow : lse_index;  // read either way; 1 is used without weights
  __syncthreads();  // row tables of chunks 0 and 1 are written

  const uint16_t* iqb = iq + ((int64_t)b * D.n_q * D.h_kv + g) * DIDX;
  const float* lzb = lse_index + (int64_t)bg * D.n_q;
  const float* wb = wsrc + (int64_t)bg * D.n_q;
  const _Float16* tk = teacher + 16 * wave + n;  // this lane's key in a (row, slot) of the teacher

  // A chunk's index rows travel through registers: lane l of wave w < NI
  // carries piece p of row RPI w + l / CPI, stored at byte 1024 w + 16 l and,
  // element by element, into the transpose.
  const int my_ri = RPI * wave + lane / CPI;
  const int my_pi = (lane % CPI) ^ (my_ri % CPI);
  u32x4 iq_next;
  auto load_rows = [&](int slot) {
    if (wave < NI) {
      const int i = max(W.row[slot][my_ri].x - (int)D.offset, 0);
      iq_next = *reinterpret_cast<const u32x4*>(iqb + (int64_t)i * D.h_kv * DIDX + 8 * my_pi);
    }
  };
  auto store_rows = [&]() {
    if (wave < NI) *reinterpret_cast<u32x4*>(IQs + 1024 * wave + 16 * lane) = iq_next;
  };
  // raw statistics of the next chunk for the lane's 8 rows 16 m + 4c + e (row
  // 0's for rows that do not exist): the student's normaliser, the row weight
  // and the teacher's weight of the lane's key
  float lz_raw[8], w_raw[8];
  _Float16 t_raw[8];
  auto stats = [&](int slot) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int r = 16 * (u >> 2) + 4 * cgrp + (u & 3);
      const int i = max(W.row[slot][r].x - (int)D.offset, 0);
      lz_raw[u] = lzb[i];
      w_raw[u] = wb[i];
      t_raw[u] = tk[W.part[slot][r] * kBk];
    }
  };

  load_rows(0);
  stats(0);
  store_rows();
  for (int c = 0; c < nch; ++c) {
    const int slot = c & (kRing - 1);
    __syncthreads();  // chunk c's rows are in LDS; chunk c + 1's table is visible
    if (wave < NI) tp_store8(IQt, iq_next, my_pi, my_ri);
    float lz2[8], wg[8], tv[8];
    int pos8[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      pos8[u] = W.row[slot][16 * (u >> 2) + 4 * cgrp + (u & 3)].x;
      lz2[u] = lz_raw[u] * kL2e;
      wg[u] = has_w ? w_raw[u] : 1.f;
      tv[u] = (float)t_raw[u];
      asm volatile("" ::"v"(lz2[u]), "v"(wg[u]), "v"(tv[u]) : "memory");  // formed before the next chunk's loads
    }
    if (wave == 0) bld_step(bd, W, ws, D1, bg, pm, c, lane);
    load_rows((c + 1) & (kRing - 1));
    stats((c + 1) & (kRing - 1));
    // Z (student), rows as M
    f32x4 z4[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      z4[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int r = 16 * mt + n;
#pragma unroll
      for (int ks = 0; ks < IKS; ++ks) {
        const u32x4 ia =
            *reinterpret_cast<const u32x4*>(IQs + r * 2 * DIDX + 16 * ((4 * ks + cgrp) ^ (r % CPI)));
        z4[mt] = mfma16(ia, ikf[ks], z4[mt]);
      }
    }
    // g = w (s - t) on every visible (row, key); 0 for rows that do not exist
    float gv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const bool vis = key_abs <= pos8[u] && key_abs < nkv;  // pos8 = -1: no row
      const float sv = __builtin_amdgcn_exp2f(__builtin_fmaf(z4[u >> 2][u & 3], kL2e, -lz2[u]));
      gv[u] = vis ? wg[u] * (sv - tv[u]) : 0.f;
    }
    const u32x4 gb = {pack_bf16x2(gv[0], gv[1]), pack_bf16x2(gv[2], gv[3]), pack_bf16x2(gv[4], gv[5]),
                      pack_bf16x2(gv[6], gv[7])};
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int r = 16 * (u >> 2) + 4 * cgrp + (u & 3);
      const int key = 16 * wave + n;
      const int sl = (key >> 3) ^ (r & 15);
      *reinterpret_cast<uint16_t*>(Ss + r * 256 + sl * 16 + 2 * (key & 7)) =
          (uint16_t)((u & 1) ? (gb[u >> 1] >> 16) : (gb[u >> 1] & 0xFFFFu));
    }
    __syncthreads();  // IQ^T and g are in LDS; the row buffers are free
    // d_ik^T += IQ^T g (M = index dims, K = the 32 rows, N = this wave's keys)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) dikT[dt] = mfma16(tp_operand(IQt, 16 * dt + n, cgrp), gb, dikT[dt]);
    // d_iq^T (dims 16w .. 16w+15 x 32 rows) = IK^T g^T over the block's keys
    if (wave < DT) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        const int r = 16 * nt + n;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const u32x4 ka = *reinterpret_cast<const u32x4*>(IKt + (16 * wave + n) * kKtP + 32 * ks + 8 * cgrp);
          const u32x4 gbv = *reinterpret_cast<const u32x4*>(Ss + r * 256 + 16 * ((4 * ks + cgrp) ^ (r & 15)));
          acc = mfma16(ka, gbv, acc);
        }
        if (W.row[slot][r].x >= 0) {
          uint16_t* dst = diq_part + W.part[slot][r] * DIDX + 16 * wave + 4 * cgrp;
          *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
        }
      }
    }
    store_rows();  // chunk c + 1's rows, read after the next barrier
  }
  // this group's share of d_ik for the wave's keys (fp32; the groups are added next)
  if (key_abs < nkv) {
    float* dst = dik_group + (((int64_t)b * D.h_kv + g) * nkv + key_abs) * DIDX;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<float4*>(dst + 16 * dt + 4 * cgrp) =
          make_float4(dikT[dt][0], dikT[dt][1], dikT[dt][2], dikT[dt][3]);
  }
}

// d_ik[b][j] = sum over groups of their shares (bf16): one thread per 4 dims.
__global__ __launch_bounds__(256) void k_kl_bwd_dik(const float* __restrict__ dik_group, uint16_t* __restrict__ dik,
                                                    Dims D) {
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int q4 = D.d_idx / 4;
  const int64_t total = (int64_t)D.B * D.n_kv * q4;
  if (id >= total) return;
  const int64_t bj = id / q4;
  const int part = (int)(id % q4);
  const int64_t b = bj / D.n_kv, j = bj % D.n_kv;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int g = 0; g < D.h_kv; ++g) {
    const float4 x = *reinterpret_cast<const float4*>(dik_group + ((b * D.h_kv + g) * D.n_kv + j) * D.d_idx + 4 * part);
    acc.x += x.x;
    acc.y += x.y;
    acc.z += x.z;
    acc.w += x.w;
  }
  *reinterpret_cast<uint2*>(dik + bj * D.d_idx + 4 * part) =
      make_uint2(pack_bf16x2(acc.x, acc.y), pack_bf16x2(acc.z, acc.w));
}

// d_iq[b][i][g] = the sum of the row's slot partials: one thread per (row, 8 dims).
__global__ __launch_bounds__(256) void k_kl_bwd_diq(const int32_t* __restrict__ block_idx,
                                                    const uint16_t* __restrict__ diq_part, uint16_t* __restrict__ diq,
                                                    Dims D) {
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int c8 = D.d_idx / 8;
  const int64_t row = id / c8;  // (b, g, i)
  if (row >= (int64_t)D.B * D.h_kv * D.n_q) return;
  const int part = (int)(id % c8);
  const int i = (int)(row % D.n_q);
  const int64_t bg = row / D.n_q;
  const int g = (int)(bg % D.h_kv), b = (int)(bg / D.h_kv);
  const int local = (int)((D.offset + i) / kBk);
  const int32_t* sel = block_idx + row * D.k;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const uint16_t* src = diq_part + row * (D.k + 1) * D.d_idx + 8 * part;  // slot s at s d_idx
  auto add = [&](uint4 x) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      acc[2 * u] += __uint_as_float(w[u] << 16);
      acc[2 * u + 1] += __uint_as_float(w[u] & 0xFFFF0000u);
    }
  };
  // the listed non-local slots in order, eight loads in flight at a time, then the local slot
  for (int s0 = 0; s0 < D.k; s0 += 8) {
    uint4 x[8];
    bool use[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      use[u] = s0 + u < D.k && nonlocal_slot(sel, s0 + u, local);
      x[u] = use[u] ? *reinterpret_cast<const uint4*>(src + (int64_t)(s0 + u) * D.d_idx) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (use[u]) add(x[u]);
  }
  add(*reinterpret_cast<const uint4*>(src + (int64_t)D.k * D.d_idx));
  uint16_t* dst = diq + (((int64_t)b * D.n_q + i) * D.h_kv + g) * D.d_idx + 8 * part;
  *reinterpret_cast<uint4*>(dst) = make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                              pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
}

}  // namespace

hipError_t launch_index_kl_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* index_q, const uint16_t* index_k,
                               const int32_t* block_idx, const float* lse, const float* lse_index, const float* wrow,
                               uint16_t* d_index_q, uint16_t* d_index_k, const AttnWs& ws, uint16_t* diq_part,
                               float* dik_group, const Dims& D, hipStream_t stream) {
  if (ws.n_groups + 1 > kMaxSrc) return hipErrorInvalidValue;  // the walk's source table
  hipError_t e = launch_gather_plan(block_idx, ws, D, stream);
  if (e == hipSuccess) e = launch_plan_sort(ws, D, stream);  // a fixed summation order
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((int64_t)D.B * D.h_kv * D.n_blk)), block(kBwdThreads);
  auto go = [&](auto didx, auto gg) {
    constexpr int DI = decltype(didx)::value, GG = decltype(gg)::value;
    hipLaunchKernelGGL((k_kl_bwd<DI, GG>), grid, block, 0, stream, q, k, index_q, index_k, lse, lse_index, wrow, ws,
                       diq_part, dik_group, D);
  };
  auto by_g = [&](auto didx) {
    switch (D.G) {
      case 4: go(didx, std::integral_constant<int, 4>{}); break;
      case 8: go(didx, std::integral_constant<int, 8>{}); break;
      case 16: go(didx, std::integral_constant<int, 16>{}); break;
      default: go(didx, std::integral_constant<int, 32>{}); break;
    }
  };
  if (D.d_idx == 128) by_g(std::integral_constant<int, 128>{}); else by_g(std::integral_constant<int, 64>{});
  const int64_t n_ik = (int64_t)D.B * D.n_kv * (D.d_idx / 4);
  hipLaunchKernelGGL(k_kl_bwd_dik, dim3((unsigned)((n_ik + 255) / 256)), dim3(256), 0, stream, dik_group, d_index_k, D);
  const int64_t n_iq = (int64_t)D.B * D.h_kv * D.n_q * (D.d_idx / 8);
  hipLaunchKernelGGL(k_kl_bwd_diq, dim3((unsigned)((n_iq + 255) / 256)), dim3(256), 0, stream, block_idx, diq_part,
                     d_index_q, D);
  return hipGetLastError();
}

hipError_t launch_index_kl_bwd_teacher(const uint16_t* index_q, const uint16_t* index_k, const int32_t* block_idx,
                                       const uint16_t* teacher, const float* lse_index, const float* wrow,
                                       uint16_t* d_index_q, uint16_t* d_index_k, const AttnWs& ws,
                                       uint16_t* diq_part, float* dik_group, const Dims& D, hipStream_t stream) {
  if (ws.n_groups + 1 > kMaxSrc) return hipErrorInvalidValue;  // the walk's source table
  hipError_t e = launch_gather_plan(block_idx, ws, D, stream);
  if (e == hipSuccess) e = launch_plan_sort(ws, D, stream);  // a fixed summation order
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((int64_t)D.B * D.h_kv * D.n_blk)), block(kBwdThreads);
  const _Float16* t = reinterpret_cast<const _Float16*>(teacher);
  if (D.d_idx == 128)
    hipLaunchKernelGGL(k_kl_bwd_t<128>, grid, block, 0, stream, index_q, index_k, t, lse_index, wrow, ws, diq_part,
                       dik_group, D);
  else
    hipLaunchKernelGGL(k_kl_bwd_t<64>, grid, block, 0, stream, index_q, index_k, t, lse_index, wrow, ws, diq_part,
                       dik_group, D);
  const int64_t n_ik = (int64_t)D.B * D.n_kv * (D.d_idx / 4);
  hipLaunchKernelGGL(k_kl_bwd_dik, dim3((unsigned)((n_ik + 255) / 256)), dim3(256), 0, stream, dik_group, d_index_k, D);
  const int64_t n_iq = (int64_t)D.B * D.h_kv * D.n_q * (D.d_idx / 8);
  hipLaunchKernelGGL(k_kl_bwd_diq, dim3((unsigned)((n_iq + 255) / 256)), dim3(256), 0, stream, block_idx, diq_part,
                     d_index_q, D);
  return hipGetLastError();
}

hipError_t launch_sparse_attn_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* block_idx,
                                  const uint16_t* out, const float* lse, const uint16_t* dout, uint16_t* dq,
                                  uint16_t* dk, uint16_t* dv, const AttnWs& ws, uint16_t* dq_part, float* delta,
                                  const Dims& D, hipStream_t stream) {
  if (ws.n_groups + 1 > kMaxSrc) return hipErrorInvalidValue;  // the walk's source table
  hipError_t e = launch_gather_plan(block_idx, ws, D, stream);
  if (e == hipSuccess) e = launch_plan_sort(ws, D, stream);  // a fixed summation order
  if (e != hipSuccess) return e;
  const int64_t pairs = (int64_t)D.B * D.n_q * D.h_q;
  hipLaunchKernelGGL(k_bwd_delta, dim3((unsigned)((pairs * 8 + 255) / 256)), dim3(256), 0, stream, out, dout, delta,
                     D);
  hipLaunchKernelGGL(k_bwd_kv<false>, dim3((unsigned)((int64_t)D.B * D.h_kv * D.n_blk)), dim3(kBwdThreads), 0,
                     stream, q, k, v, dout, lse, delta, ws, dq_part, dk, dv, D);
  const int64_t threads = (int64_t)D.B * D.h_kv * D.n_q * D.G * 16;
  hipLaunchKernelGGL(k_bwd_dq_merge, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, block_idx,
                     dq_part, dq, D);
  return hipGetLastError();
}

}  // namespace msa
