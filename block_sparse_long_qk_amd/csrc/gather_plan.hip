// Gather plan of the KV-outer attention (page "MiniMax 发布 MSA 稀疏注意力方法，开源推理
// 内核并推出 MiniMax-M3 模型", section 内核协同设计: iterate over KV blocks and gather
// the query positions that selected each one).
//
// Input: block_idx rows (one per sequence, group, query).  Output: for every
// bin (sequence b, group g, query chunk group c of kGroupRows rows, block t)
// the list of row-slot ids i*k + s of the rows in c that picked t as a
// non-local block, the lists stored back to back in (b, g, c, t) order, and a
// tile list cutting each list into runs of `pt` query positions.  Binning by
// chunk group keeps the query rows that consecutive tiles gather within
// kGroupRows positions.
//
// A counting sort without global atomics:
//   1. hist:  one workgroup per chunk of kChunkRows rows of one (b, g) counts its
//             entries per block in LDS and writes the chunk's histogram;
//   2. colscan: per bin, exclusive scan of its chunks' histograms (the chunk's
//             start inside the list) and the list length;
//   3. scan:  exclusive scans of the list lengths and of their tile counts over
//             all bins (two-level: block sums, one-workgroup scan, apply);
//   4. fill:  each chunk workgroup re-reads its rows and scatters row-slot ids
//             with LDS cursors into the tile-major list: bin b owns list slots
//             [tile_off[b] * pt, tile_off[b+1] * pt), so tile j's rows are
//             list[j * pt .. j * pt + pt);
//   5. tiles: the bin of every tile, and -1 in the unused slots of each bin's
//             last tile.
// Step 4 also marks every slot that carries no partial (a padding entry, a
// repeat, the local block or a block past it) with a log-sum-exp of -inf, so
// that the merge needs no block_idx.
// Entries inside one list appear in no fixed order; every row's attention is
// independent of the other rows of its tile, so results do not depend on it.
#include <algorithm>

#include "launch.h"

namespace msa {
namespace {

constexpr int kScanPer = 4096;  // elements per workgroup in the two-level scan

__global__ __launch_bounds__(256) void k_plan_hist(const int32_t* __restrict__ block_idx,
                                                   int32_t* __restrict__ hist, Dims D, int32_t n_ch) {
  extern __shared__ int32_t lh[];  // [n_blk]
  const int ch = blockIdx.x, bg = blockIdx.y;
  for (int t = threadIdx.x; t < D.n_blk; t += blockDim.x) lh[t] = 0;
  __syncthreads();
  const int b = bg / D.h_kv;
  const int64_t off_b = seq_offset(D, b);
  const int i0 = ch * kChunkRows, i1 = min(seq_nq(D, b), i0 + kChunkRows);
  for (int i = i0 + (int)threadIdx.x; i < i1; i += blockDim.x) {
    const int local = (int)((off_b + i) / kBk);
    const int32_t* row = block_idx + ((int64_t)bg * D.n_q + i) * D.k;
    for (int s = 0; s < D.k; ++s)
      if (nonlocal_slot(row, s, local)) atomicAdd(&lh[row[s]], 1);
  }
  __syncthreads();
  int32_t* dst = hist + ((int64_t)bg * n_ch + ch) * D.n_blk;
  for (int t = threadIdx.x; t < D.n_blk; t += blockDim.x) dst[t] = lh[t];
}

// hist[bg][ch][t] <- exclusive prefix over the chunks of ch's group;
// cnt[(bg*n_cg + cg)*n_blk + t] <- the group's total.
__global__ void k_plan_colscan(int32_t* __restrict__ hist, int32_t* __restrict__ cnt, Dims D, int32_t n_ch) {
  const int n_cg = (n_ch + kGroupChunks - 1) / kGroupChunks;
  const int64_t nbins = (int64_t)D.B * D.h_kv * n_cg * D.n_blk;
  for (int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; x < nbins; x += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = x % D.n_blk;
    const int64_t cg = (x / D.n_blk) % n_cg;
    const int64_t bg = x / ((int64_t)D.n_blk * n_cg);
    int32_t acc = 0;
    const int ch1 = min(n_ch, (int)(cg + 1) * kGroupChunks);
    for (int ch = (int)cg * kGroupChunks; ch < ch1; ++ch) {
      int32_t* h = hist + (bg * n_ch + ch) * D.n_blk + t;
      const int32_t v = *h;
      *h = acc;
      acc += v;
    }
    cnt[x] = acc;
  }
}

__device__ __forceinline__ int32_t tiles_of(int32_t c, int32_t pt) { return (c + pt - 1) / pt; }

// Block-wide inclusive scan of two values (256 threads).
__device__ __forceinline__ void block_scan2(int32_t& a, int32_t& b, int32_t* sa, int32_t* sb) {
  const int tid = threadIdx.x;
  sa[tid] = a;
  sb[tid] = b;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const int32_t ya = tid >= o ? sa[tid - o] : 0, yb = tid >= o ? sb[tid - o] : 0;
    __syncthreads();
    sa[tid] += ya;
    sb[tid] += yb;
    __syncthreads();
  }
  a = sa[tid];
  b = sb[tid];
}

__global__ __launch_bounds__(256) void k_scan_reduce(const int32_t* __restrict__ cnt, int32_t* __restrict__ bsum,
                                                     int64_t n, int32_t pt) {
  __shared__ int32_t sa[256], sb[256];
  const int64_t a0 = (int64_t)blockIdx.x * kScanPer;
  int32_t e = 0, t = 0;
  for (int64_t x = a0 + threadIdx.x; x < min(n, a0 + kScanPer); x += 256) {
    e += cnt[x];
    t += tiles_of(cnt[x], pt);
  }
  block_scan2(e, t, sa, sb);
  if (threadIdx.x == 255) {
    bsum[2 * blockIdx.x] = e;
    bsum[2 * blockIdx.x + 1] = t;
  }
}

// One workgroup: exclusive scan of the (edges, tiles) block sums in place;
// writes the grand totals to off[n] and tile_off[n], and clears the work
// counters of the attention kernels that follow the plan.
__global__ __launch_bounds__(256) void k_scan_blocks(int32_t* __restrict__ bsum, int32_t nb, int32_t* __restrict__ off,
                                                     int32_t* __restrict__ tile_off, int64_t n,
                                                     int32_t* __restrict__ ctr) {
  __shared__ int32_t sa[256], sb[256];
  if (threadIdx.x < kWorkCounters) ctr[threadIdx.x] = 0;
  const int per = (nb + 255) / 256;
  const int a0 = threadIdx.x * per, a1 = min(nb, a0 + per);
  int32_t e = 0, t = 0;
  for (int x = a0; x < a1; ++x) {
    e += bsum[2 * x];
    t += bsum[2 * x + 1];
  }
  const int32_t e_own = e, t_own = t;
  block_scan2(e, t, sa, sb);
  int32_t re = e - e_own, rt = t - t_own;
  for (int x = a0; x < a1; ++x) {
    const int32_t ve = bsum[2 * x], vt = bsum[2 * x + 1];
    bsum[2 * x] = re;
    bsum[2 * x + 1] = rt;
    re += ve;
    rt += vt;
  }
  if (threadIdx.x == 255) {
    off[n] = e;
    tile_off[n] = t;
  }
}

__global__ __launch_bounds__(256) void k_scan_apply(const int32_t* __restrict__ cnt, const int32_t* __restrict__ bsum,
                                                    int32_t* __restrict__ off, int32_t* __restrict__ tile_off,
                                                    int64_t n, int32_t pt) {
  __shared__ int32_t sa[256], sb[256];
  const int64_t a0 = (int64_t)blockIdx.x * kScanPer;
  constexpr int kPer = kScanPer / 256;  // contiguous elements per thread
  const int64_t b0 = a0 + (int64_t)threadIdx.x * kPer;
  int32_t e = 0, t = 0;
  for (int u = 0; u < kPer; ++u) {
    const int64_t x = b0 + u;
    if (x < n) {
      e += cnt[x];
      t += tiles_of(cnt[x], pt);
    }
  }
  const int32_t e_own = e, t_own = t;
  block_scan2(e, t, sa, sb);
  int32_t re = bsum[2 * blockIdx.x] + e - e_own, rt = bsum[2 * blockIdx.x + 1] + t - t_own;
  for (int u = 0; u < kPer; ++u) {
    const int64_t x = b0 + u;
    if (x < n) {
      off[x] = re;
      tile_off[x] = rt;
      re += cnt[x];
      rt += tiles_of(cnt[x], pt);
    }
  }
}

__global__ __launch_bounds__(256) void k_plan_fill(const int32_t* __restrict__ block_idx,
                                                   const int32_t* __restrict__ hist,
                                                   const int32_t* __restrict__ tile_off, int2* __restrict__ list,
                                                   float* __restrict__ part_lse, Dims D, int32_t n_ch) {
  extern __shared__ int32_t cursor[];  // [n_blk]
  const int ch = blockIdx.x, bg = blockIdx.y;
  const int n_cg = (n_ch + kGroupChunks - 1) / kGroupChunks;
  const int32_t* h = hist + ((int64_t)bg * n_ch + ch) * D.n_blk;
  const int32_t* o = tile_off + ((int64_t)bg * n_cg + ch / kGroupChunks) * D.n_blk;
  for (int t = threadIdx.x; t < D.n_blk; t += blockDim.x) cursor[t] = o[t] * D.pt + h[t];
  __syncthreads();
  const int b = bg / D.h_kv;
  const int64_t off_b = seq_offset(D, b);
  const int i0 = ch * kChunkRows, i1 = min(seq_nq(D, b), i0 + kChunkRows);
  const int bin0 = (bg * n_cg + ch / kGroupChunks) * D.n_blk;  // bin of block 0 in this chunk's group
  const float4 neg4 = make_float4(-__builtin_huge_valf(), -__builtin_huge_valf(), -__builtin_huge_valf(),
                                  -__builtin_huge_valf());
  for (int i = i0 + (int)threadIdx.x; i < i1; i += blockDim.x) {
    const int local = (int)((off_b + i) / kBk);
    const int32_t* row = block_idx + ((int64_t)bg * D.n_q + i) * D.k;
    float* lse_row = part_lse + ((int64_t)bg * D.n_q + i) * (D.k + 1) * D.G;
    for (int s = 0; s < D.k; ++s) {
      if (nonlocal_slot(row, s, local)) {
        list[atomicAdd(&cursor[row[s]], 1)] = make_int2(i * D.k + s, bin0 + row[s]);
      } else if ((D.G & 3) == 0) {  // 16-byte aligned runs of G floats
        float4* dst = reinterpret_cast<float4*>(lse_row + s * D.G);
        for (int h = 0; h < D.G / 4; ++h) dst[h] = neg4;
      } else {
        for (int h = 0; h < D.G; ++h) lse_row[s * D.G + h] = -__builtin_huge_valf();
      }
    }
  }
}

// The padding entries of each bin's last tile: the empty id -1 and the bin
// (every entry of a tile carries its bin; step 4 wrote the others).
__global__ void k_plan_tiles(const int32_t* __restrict__ cnt, const int32_t* __restrict__ tile_off,
                             int2* __restrict__ list, int64_t n, int32_t pt) {
  for (int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; x < n; x += (int64_t)gridDim.x * blockDim.x) {
    const int c = cnt[x];
    const int nt = tiles_of(c, pt);
    int2* l = list + (int64_t)tile_off[x] * pt;
    for (int sl = c; sl < nt * pt; ++sl) l[sl] = make_int2(-1, (int32_t)x);
  }
}

// Canonical order of every bin's entries: ascending row-slot id.  The fill
// places a bin's entries in the order the waves of a workgroup reach their
// atomics, which can change from run to run; the attention forward does not
// care (each entry is computed on its own), but sums over a bin's rows (the
// backward passes) are reproducible only in a fixed order.  One workgroup
// sorts one bin at a time in LDS (bitonic, padded to a power of two); a bin
// holds at most one entry per row of its query group.
constexpr int kSortCap = kChunkRows * kGroupChunks;
__global__ __launch_bounds__(256) void k_plan_sort(const int32_t* __restrict__ cnt, const int32_t* __restrict__ tile_off,
                                                   int2* __restrict__ list, int64_t n_bins, int32_t pt) {
  __shared__ int32_t key[kSortCap];
  for (int64_t bin = blockIdx.x; bin < n_bins; bin += gridDim.x) {
    const int c = min(cnt[bin], kSortCap);  // uniform over the workgroup
    if (c <= 1) continue;
    int2* l = list + (int64_t)tile_off[bin] * pt;
    int n = 2;
    while (n < c) n <<= 1;
    for (int i = threadIdx.x; i < n; i += blockDim.x) key[i] = i < c ? l[i].x : 0x7FFFFFFF;
    __syncthreads();
    for (int k = 2; k <= n; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = threadIdx.x; i < n; i += blockDim.x) {
          const int o = i ^ j;
          if (o > i) {
            const int a = key[i], b = key[o];
            if ((a > b) == ((i & k) == 0)) {
              key[i] = b;
              key[o] = a;
            }
          }
        }
        __syncthreads();
      }
    }
    for (int i = threadIdx.x; i < c; i += blockDim.x) l[i].x = key[i];
    __syncthreads();  // key[] is free for the next bin
  }
}

unsigned grid_for(int64_t n, int threads) {
  int64_t g = (n + threads - 1) / threads;
  if (g < 1) g = 1;
  if (g > 65536) g = 65536;
  return (unsigned)g;
}

}  // namespace

int64_t plan_chunks(const Dims& D) { return (D.n_q + kChunkRows - 1) / kChunkRows; }

int64_t plan_groups(const Dims& D) { return (plan_chunks(D) + kGroupChunks - 1) / kGroupChunks; }

int64_t plan_bins(const Dims& D) { return (int64_t)D.B * D.h_kv * plan_groups(D) * D.n_blk; }

int64_t plan_scan_blocks(const Dims& D) { return (plan_bins(D) + kScanPer - 1) / kScanPer; }

hipError_t launch_gather_plan(const int32_t* block_idx, const AttnWs& ws, const Dims& D, hipStream_t stream) {
  const int64_t nbgt = plan_bins(D);
  const int n_ch = (int)plan_chunks(D);
  const int nb = (int)plan_scan_blocks(D);
  const size_t lds = sizeof(int32_t) * D.n_blk;
  dim3 cgrid(n_ch, D.B * D.h_kv);
  hipLaunchKernelGGL(k_plan_hist, cgrid, dim3(256), lds, stream, block_idx, ws.hist, D, n_ch);
  mark("k_plan_hist", stream);
  hipLaunchKernelGGL(k_plan_colscan, dim3(grid_for(nbgt, 256)), dim3(256), 0, stream, ws.hist, ws.cnt, D, n_ch);
  mark("k_plan_colscan", stream);
  hipLaunchKernelGGL(k_scan_reduce, dim3(nb), dim3(256), 0, stream, ws.cnt, ws.bsum, nbgt, D.pt);
  mark("k_scan_reduce", stream);
  hipLaunchKernelGGL(k_scan_blocks, dim3(1), dim3(256), 0, stream, ws.bsum, nb, ws.off, ws.tile_off, nbgt,
                     ws.ctr);
  mark("k_scan_blocks", stream);
  hipLaunchKernelGGL(k_scan_apply, dim3(nb), dim3(256), 0, stream, ws.cnt, ws.bsum, ws.off, ws.tile_off, nbgt, D.pt);
  mark("k_scan_apply", stream);
  hipLaunchKernelGGL(k_plan_fill, cgrid, dim3(256), lds, stream, block_idx, ws.hist, ws.tile_off, ws.list,
                     ws.part_lse, D, n_ch);
  mark("k_plan_fill", stream);
  hipLaunchKernelGGL(k_plan_tiles, dim3(grid_for(nbgt, 256)), dim3(256), 0, stream, ws.cnt, ws.tile_off, ws.list,
                     nbgt, D.pt);
  mark("k_plan_tiles", stream);
  return hipGetLastError();
}

namespace {

// n_seg runs of `words` 32-bit words, run s read at src + s * src_pitch and
// written at dst + s * dst_pitch; `parts` workgroups share each run.
__global__ __launch_bounds__(256) void k_copy_runs(const uint32_t* __restrict__ src, int64_t src_pitch,
                                                   uint32_t* __restrict__ dst, int64_t dst_pitch, int64_t words,
                                                   int parts) {
  const int64_t seg = blockIdx.x / parts, part = blockIdx.x % parts;
  const int64_t per = (words + parts - 1) / parts;
  const int64_t i0 = part * per, i1 = min(words, i0 + per);
  const uint32_t* s = src + seg * src_pitch;
  uint32_t* d = dst + seg * dst_pitch;
  for (int64_t i = i0 + threadIdx.x; i < i1; i += 256) d[i] = s[i];
}

}  // namespace

hipError_t launch_copy_runs(const void* src, int64_t src_pitch, void* dst, int64_t dst_pitch, int64_t words,
                            int64_t n_seg, hipStream_t stream) {
  if (words <= 0 || n_seg <= 0) return hipSuccess;
  const int parts = (int)std::min<int64_t>(std::max<int64_t>(1, words / 8192), 256);
  hipLaunchKernelGGL(k_copy_runs, dim3((unsigned)(n_seg * parts)), dim3(256), 0, stream,
                     static_cast<const uint32_t*>(src), src_pitch, static_cast<uint32_t*>(dst), dst_pitch, words,
                     parts);
  mark("k_copy_runs", stream);
  return hipGetLastError();
}

hipError_t launch_plan_sort(const AttnWs& ws, const Dims& D, hipStream_t stream) {
  const int64_t nbgt = plan_bins(D);
  hipLaunchKernelGGL(k_plan_sort, dim3(grid_for(nbgt, 1)), dim3(256), 0, stream, ws.cnt, ws.tile_off, ws.list, nbgt,
                     D.pt);
  mark("k_plan_sort", stream);
  return hipGetLastError();
}

}  // namespace msa
