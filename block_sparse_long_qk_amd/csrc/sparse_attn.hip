// Main Branch: exact softmax attention over the selected blocks.
//
// Page "MiniMax 发布 MSA 稀疏注意力方法，开源推理内核并推出 MiniMax-M3 模型":
// section 两个分支如何工作 (gather the causally visible tokens of the selected
// blocks; scaled dot-product softmax per query head; the group's heads share
// the block set) and section 内核协同设计 (iterate over KV blocks rather than
// queries, packing gathered query positions into 128x128 score tiles; attention
// and merge run as two separate stages).
//
// Stage A, gather plan: for every (sequence, group, block) the list of query
//   rows that selected it as a non-local block (histogram, scan, scatter), cut
//   into tiles of `pt` positions (pt * G <= 128 rows).
// Stage B, non-local tiles (KV-outer): one workgroup per tile loads the 128-key
//   K block and V block once into LDS, gathers the tile's query rows and
//   computes S^T = K Q^T and O^T = V^T P^T with 32x32x16 bf16 MFMA.  A
//   non-local block lies wholly before the query, so no mask is needed.  Each
//   (row, slot) writes a normalised bf16 partial and its base-2 log-sum-exp.
// Stage C, local tiles + merge: one workgroup per run of `pt` consecutive
//   positions, which share their local block; it computes that block with the
//   causal mask, then merges the row's partials (LSE weighting) and writes the
//   bf16 output and the natural-log lse.
//
// Lane layout: a wave owns 32 rows (one MFMA n-tile); lane l holds column
// l % 32, so all softmax statistics of a row live in one lane pair (l, l ^ 32).
#include "launch.h"

namespace msa {
namespace {

constexpr int KP = kHeadDim + 8;   // LDS pitch of K rows (bf16): 16-byte pad
constexpr int VP = kBk + 4;        // LDS pitch of V^T rows (bf16): 8-byte pad

// Is slot s of a block_idx row a non-local block with its own partial?
// (Rows are ascending; a repeated entry is ignored; the local block and
// anything past it carry no partial.)
__device__ __forceinline__ bool nonlocal_slot(const int32_t* row, int s, int local) {
  const int t = row[s];
  return t >= 0 && t < local && (s == 0 || row[s - 1] != t);
}

__global__ void k_fill_zero(int32_t* __restrict__ p, int64_t n) {
  for (int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; x < n; x += (int64_t)gridDim.x * blockDim.x)
    p[x] = 0;
}

__global__ void k_plan_count(const int32_t* __restrict__ block_idx, int32_t* __restrict__ cnt, Dims D) {
  const int64_t nrows = (int64_t)D.B * D.h_kv * D.n_q;
  for (int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; r < nrows; r += (int64_t)gridDim.x * blockDim.x) {
    const int64_t bg = r / D.n_q;
    const int i = (int)(r % D.n_q);
    const int local = (int)((D.offset + i) / kBk);
    const int32_t* row = block_idx + r * D.k;
    for (int s = 0; s < D.k; ++s)
      if (nonlocal_slot(row, s, local)) atomicAdd(&cnt[bg * D.n_blk + row[s]], 1);
  }
}

// Exclusive scans of cnt and of ceil(cnt / pt) by one workgroup of 1024 threads.
__global__ __launch_bounds__(1024) void k_plan_scan(const int32_t* __restrict__ cnt, int32_t* __restrict__ off,
                                                    int32_t* __restrict__ tile_off, int64_t n, int32_t pt) {
  __shared__ int32_t s_e[1024], s_t[1024];
  const int tid = threadIdx.x;
  const int64_t chunk = (n + 1023) / 1024;
  const int64_t a = tid * chunk, z = min(n, a + chunk);
  int32_t se = 0, st = 0;
  for (int64_t x = a; x < z; ++x) {
    se += cnt[x];
    st += (cnt[x] + pt - 1) / pt;
  }
  s_e[tid] = se;
  s_t[tid] = st;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {  // Hillis-Steele inclusive scan
    const int32_t ye = tid >= o ? s_e[tid - o] : 0, yt = tid >= o ? s_t[tid - o] : 0;
    __syncthreads();
    s_e[tid] += ye;
    s_t[tid] += yt;
    __syncthreads();
  }
  int32_t re = s_e[tid] - se, rt = s_t[tid] - st;
  for (int64_t x = a; x < z; ++x) {
    off[x] = re;
    tile_off[x] = rt;
    re += cnt[x];
    rt += (cnt[x] + pt - 1) / pt;
  }
  if (tid == 1023) {
    off[n] = s_e[1023];
    tile_off[n] = s_t[1023];
  }
}

__global__ void k_plan_fill(const int32_t* __restrict__ block_idx, int32_t* __restrict__ cursor,
                            const int32_t* __restrict__ off, int32_t* __restrict__ list, Dims D) {
  const int64_t nrows = (int64_t)D.B * D.h_kv * D.n_q;
  for (int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; r < nrows; r += (int64_t)gridDim.x * blockDim.x) {
    const int64_t bg = r / D.n_q;
    const int i = (int)(r % D.n_q);
    const int local = (int)((D.offset + i) / kBk);
    const int32_t* row = block_idx + r * D.k;
    for (int s = 0; s < D.k; ++s) {
      if (!nonlocal_slot(row, s, local)) continue;
      const int64_t bgt = bg * D.n_blk + row[s];
      const int at = atomicAdd(&cursor[bgt], 1);
      list[off[bgt] + at] = i * D.k + s;
    }
  }
}

__global__ void k_plan_tiles(const int32_t* __restrict__ cnt, const int32_t* __restrict__ tile_off,
                             int32_t* __restrict__ tile_desc, int64_t n, int32_t pt) {
  for (int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; x < n; x += (int64_t)gridDim.x * blockDim.x) {
    const int nt = (cnt[x] + pt - 1) / pt;
    for (int j = 0; j < nt; ++j) {
      tile_desc[2 * (int64_t)(tile_off[x] + j)] = (int32_t)x;
      tile_desc[2 * (int64_t)(tile_off[x] + j) + 1] = j * pt;
    }
  }
}

// Stage one 128-key block of K (row-major, padded) and V (transposed) into LDS.
// Keys at or past n_valid are zero-filled.
__device__ __forceinline__ void stage_kv(uint16_t* Ks, uint16_t* Vt, const uint16_t* __restrict__ kb,
                                         const uint16_t* __restrict__ vb, int n_valid) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < 8; ++u) {  // K: 2048 chunks of 16 B
    const int c = tid + 256 * u;
    const int key = c >> 4, oc = c & 15;
    const uint4 x = key < n_valid ? *reinterpret_cast<const uint4*>(kb + key * kHeadDim + oc * 8)
                                  : make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4*>(Ks + key * KP + oc * 8) = x;
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {  // V: 512 units of 4 keys x 8 dims, written transposed
    const int c = tid + 256 * u;
    const int kq = c >> 4, od = c & 15;
    uint4 r[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int key = kq * 4 + q;
      r[q] = key < n_valid ? *reinterpret_cast<const uint4*>(vb + key * kHeadDim + od * 8) : make_uint4(0, 0, 0, 0);
    }
    const uint32_t* w[4] = {reinterpret_cast<const uint32_t*>(&r[0]), reinterpret_cast<const uint32_t*>(&r[1]),
                            reinterpret_cast<const uint32_t*>(&r[2]), reinterpret_cast<const uint32_t*>(&r[3])};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int sh = (e & 1) * 16;
      const uint32_t v0 = (w[0][e >> 1] >> sh) & 0xFFFFu, v1 = (w[1][e >> 1] >> sh) & 0xFFFFu;
      const uint32_t v2 = (w[2][e >> 1] >> sh) & 0xFFFFu, v3 = (w[3][e >> 1] >> sh) & 0xFFFFu;
      *reinterpret_cast<uint2*>(Vt + (od * 8 + e) * VP + kq * 4) = make_uint2(v0 | (v1 << 16), v2 | (v3 << 16));
    }
  }
}

__device__ __forceinline__ void load_q_row(uint4 (&qb)[8], const uint16_t* __restrict__ qrow, bool valid, int half) {
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
    qb[ks] = valid ? *reinterpret_cast<const uint4*>(qrow + 16 * ks + 8 * half) : make_uint4(0, 0, 0, 0);
}

// One wave, 32 query rows x one 128-key block.  Returns the unnormalised O^T
// accumulators, the row max m2 and sum l in base-2 units (score*scale*log2 e).
// With `masked`, key key0+j is dropped for rows whose position p < key0+j.
__device__ __forceinline__ void attn_block(const uint16_t* Ks, const uint16_t* Vt, const uint4 (&qb)[8], int lane,
                                           float scale_log2, bool masked, int64_t key0, int64_t p, f32x16 (&o)[4],
                                           float& m2, float& l) {
  const float NEG_INF = -__builtin_huge_valf();
  const int col = lane & 31, half = lane >> 5;
  f32x16 s[4];
#pragma unroll
  for (int T = 0; T < 4; ++T) {
    s[T] = f32x16{};
    const uint16_t* krow = Ks + (32 * T + col) * KP + 8 * half;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) s[T] = mfma_32x32x16(*reinterpret_cast<const uint4*>(krow + 16 * ks), qb[ks], s[T]);
  }
  float mx = NEG_INF;
#pragma unroll
  for (int T = 0; T < 4; ++T) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float x = s[T][e] * scale_log2;
      if (masked && key0 + 32 * T + acc_row(e, lane) > p) x = NEG_INF;
      s[T][e] = x;
      mx = fmaxf(mx, x);
    }
  }
  mx = fmaxf(mx, wave_xor32(mx));
  const float mref = mx == NEG_INF ? 0.f : mx;  // rows with nothing visible (padding rows)
  float sum = 0.f;
#pragma unroll
  for (int T = 0; T < 4; ++T) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float pe = __builtin_amdgcn_exp2f(s[T][e] - mref);
      s[T][e] = pe;
      sum += pe;
    }
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
  m2 = mx;
  l = sum;
}

__global__ __launch_bounds__(256) void k_attn_nonlocal(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                       const uint16_t* __restrict__ v, AttnWs ws, Dims D) {
  __shared__ __align__(16) uint16_t Ks[kBk * KP];
  __shared__ __align__(16) uint16_t Vt[kHeadDim * VP];
  const int64_t nbgt = (int64_t)D.B * D.h_kv * D.n_blk;
  const int tile = blockIdx.x;
  if (tile >= ws.tile_off[nbgt]) return;  // uniform over the workgroup
  const int bgt = ws.tile_desc[2 * (int64_t)tile];
  const int start = ws.tile_desc[2 * (int64_t)tile + 1];
  const int t = bgt % D.n_blk;
  const int bg = bgt / D.n_blk;
  const int g = bg % D.h_kv, b = bg / D.h_kv;
  const int npos = min(D.pt, ws.cnt[bgt] - start);

  const int64_t kv0 = ((int64_t)bg * D.n_kv + (int64_t)t * kBk) * kHeadDim;
  stage_kv(Ks, Vt, k + kv0, v + kv0, kBk);

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 31, half = lane >> 5;
  const int r = wave * 32 + col;
  const int ps = r / D.G, hh = r % D.G;
  const bool valid = ps < npos;
  int i = 0, s = 0;
  if (valid) {
    const int e = ws.list[ws.off[bgt] + start + ps];
    i = e / D.k;
    s = e % D.k;
  }
  uint4 qb[8];
  load_q_row(qb, q + (((int64_t)b * D.n_q + i) * D.h_q + g * D.G + hh) * kHeadDim, valid, half);
  __syncthreads();
  if (wave * 32 >= npos * D.G) return;  // no rows for this wave

  f32x16 o[4];
  float m2, l;
  attn_block(Ks, Vt, qb, lane, D.scale_log2, false, 0, 0, o, m2, l);
  if (!valid) return;
  const int64_t pidx = ((((int64_t)bg * D.n_q + i) * D.k + s) * D.G + hh);
  if (half == 0) ws.part_lse[pidx] = m2 + __log2f(l);
  const float inv = 1.f / l;
  uint16_t* dst = ws.part_o + pidx * kHeadDim;
#pragma unroll
  for (int Dt = 0; Dt < 4; ++Dt) {
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d0 = 32 * Dt + 8 * i4 + 4 * half;
      const uint2 w = make_uint2(pack_bf16x2(o[Dt][4 * i4 + 0] * inv, o[Dt][4 * i4 + 1] * inv),
                                 pack_bf16x2(o[Dt][4 * i4 + 2] * inv, o[Dt][4 * i4 + 3] * inv));
      *reinterpret_cast<uint2*>(dst + d0) = w;
    }
  }
}

__global__ __launch_bounds__(256) void k_attn_local_merge(const uint16_t* __restrict__ q,
                                                          const uint16_t* __restrict__ k,
                                                          const uint16_t* __restrict__ v,
                                                          const int32_t* __restrict__ block_idx, AttnWs ws,
                                                          uint16_t* __restrict__ out, float* __restrict__ lse_out,
                                                          Dims D, int64_t a0) {
  __shared__ __align__(16) uint16_t Ks[kBk * KP];
  __shared__ __align__(16) uint16_t Vt[kHeadDim * VP];
  const int bg = blockIdx.y;
  const int g = bg % D.h_kv, b = bg / D.h_kv;
  const int64_t p0 = (a0 + blockIdx.x) * (int64_t)D.pt;  // first position of this run
  const int lblk = (int)(p0 / kBk);
  const int64_t key0 = (int64_t)lblk * kBk;
  const int n_valid = (int)min((int64_t)kBk, (int64_t)D.n_kv - key0);

  const int64_t kv0 = ((int64_t)bg * D.n_kv + key0) * kHeadDim;
  stage_kv(Ks, Vt, k + kv0, v + kv0, n_valid);

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 31, half = lane >> 5;
  const int r = wave * 32 + col;
  const int ps = r / D.G, hh = r % D.G;
  const int64_t p = p0 + ps;
  const bool valid = ps < D.pt && p >= D.offset && p < D.offset + D.n_q;
  const int i = valid ? (int)(p - D.offset) : 0;
  uint4 qb[8];
  load_q_row(qb, q + (((int64_t)b * D.n_q + i) * D.h_q + g * D.G + hh) * kHeadDim, valid, half);
  __syncthreads();
  if (wave * 32 >= D.pt * D.G) return;

  f32x16 o[4];
  float m2, l;
  attn_block(Ks, Vt, qb, lane, D.scale_log2, true, key0, valid ? p : -1, o, m2, l);
  if (!valid) return;

  // merge with the partials of the row's non-local blocks
  const float lse_loc = m2 + __log2f(l);
  const int32_t* row = block_idx + ((int64_t)bg * D.n_q + i) * D.k;
  const int64_t pbase = (((int64_t)bg * D.n_q + i) * D.k) * D.G + hh;  // + s * G
  float mtot = lse_loc;
  for (int s = 0; s < D.k; ++s)
    if (nonlocal_slot(row, s, lblk)) mtot = fmaxf(mtot, ws.part_lse[pbase + (int64_t)s * D.G]);
  float wsum = __builtin_amdgcn_exp2f(lse_loc - mtot);
  for (int s = 0; s < D.k; ++s)
    if (nonlocal_slot(row, s, lblk)) wsum += __builtin_amdgcn_exp2f(ws.part_lse[pbase + (int64_t)s * D.G] - mtot);
  const float lse_tot = mtot + __log2f(wsum);
  const float c_loc = __builtin_amdgcn_exp2f(lse_loc - lse_tot) / l;
#pragma unroll
  for (int Dt = 0; Dt < 4; ++Dt) o[Dt] *= c_loc;
  for (int s = 0; s < D.k; ++s) {
    if (!nonlocal_slot(row, s, lblk)) continue;
    const int64_t pidx = pbase + (int64_t)s * D.G;
    const float c = __builtin_amdgcn_exp2f(ws.part_lse[pidx] - lse_tot);
    const uint16_t* src = ws.part_o + pidx * kHeadDim;
#pragma unroll
    for (int Dt = 0; Dt < 4; ++Dt) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const uint2 w = *reinterpret_cast<const uint2*>(src + 32 * Dt + 8 * i4 + 4 * half);
        o[Dt][4 * i4 + 0] += c * bf16_to_f32(w.x & 0xFFFFu);
        o[Dt][4 * i4 + 1] += c * bf16_to_f32(w.x >> 16);
        o[Dt][4 * i4 + 2] += c * bf16_to_f32(w.y & 0xFFFFu);
        o[Dt][4 * i4 + 3] += c * bf16_to_f32(w.y >> 16);
      }
    }
  }
  uint16_t* dst = out + (((int64_t)b * D.n_q + i) * D.h_q + g * D.G + hh) * kHeadDim;
#pragma unroll
  for (int Dt = 0; Dt < 4; ++Dt) {
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d0 = 32 * Dt + 8 * i4 + 4 * half;
      *reinterpret_cast<uint2*>(dst + d0) = make_uint2(pack_bf16x2(o[Dt][4 * i4 + 0], o[Dt][4 * i4 + 1]),
                                                       pack_bf16x2(o[Dt][4 * i4 + 2], o[Dt][4 * i4 + 3]));
    }
  }
  if (lse_out && half == 0)
    lse_out[((int64_t)b * D.h_q + g * D.G + hh) * D.n_q + i] = lse_tot * 0.69314718055994531f;
}

unsigned grid_for(int64_t n, int threads) {
  int64_t g = (n + threads - 1) / threads;
  if (g < 1) g = 1;
  if (g > 65536) g = 65536;
  return (unsigned)g;
}

}  // namespace

hipError_t launch_sparse_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* block_idx,
                              uint16_t* out, float* lse, const AttnWs& ws, const Dims& D, hipStream_t stream) {
  const int64_t nbgt = (int64_t)D.B * D.h_kv * D.n_blk;
  const int64_t nrows = (int64_t)D.B * D.h_kv * D.n_q;
  // cnt and cursor are adjacent in the workspace: clear both with one fill kernel
  hipLaunchKernelGGL(k_fill_zero, dim3(grid_for(2 * nbgt, 256)), dim3(256), 0, stream, ws.cnt, 2 * nbgt);
  hipLaunchKernelGGL(k_plan_count, dim3(grid_for(nrows, 256)), dim3(256), 0, stream, block_idx, ws.cnt, D);
  hipLaunchKernelGGL(k_plan_scan, dim3(1), dim3(1024), 0, stream, ws.cnt, ws.off, ws.tile_off, nbgt, D.pt);
  hipLaunchKernelGGL(k_plan_fill, dim3(grid_for(nrows, 256)), dim3(256), 0, stream, block_idx, ws.cursor, ws.off,
                     ws.list, D);
  hipLaunchKernelGGL(k_plan_tiles, dim3(grid_for(nbgt, 256)), dim3(256), 0, stream, ws.cnt, ws.tile_off,
                     ws.tile_desc, nbgt, D.pt);
  if (ws.max_tiles > 0)
    hipLaunchKernelGGL(k_attn_nonlocal, dim3((unsigned)ws.max_tiles), dim3(256), 0, stream, q, k, v, ws, D);
  const int64_t a0 = D.offset / D.pt;
  const int64_t a1 = (D.offset + D.n_q - 1) / D.pt;
  hipLaunchKernelGGL(k_attn_local_merge, dim3((unsigned)(a1 - a0 + 1), (unsigned)(D.B * D.h_kv)), dim3(256), 0,
                     stream, q, k, v, block_idx, ws, out, lse, D, a0);
  return hipGetLastError();
}

}  // namespace msa
