// Index Branch, part 1: index scores against the shared index-key head with
// the block max-pool fused into the MFMA epilogue.
//
// Page "MiniMax 发布 MSA 稀疏注意力方法，开源推理内核并推出 MiniMax-M3 模型", section
// 两个分支如何工作: one index-query head per GQA group, one shared index-key head;
// the visible key tokens are scored and the scores max-pooled to blocks.
//
// All groups share the index keys, so the (query, group) rows of one sequence
// form a single GEMM [n_q*h_kv, d_idx] x [d_idx, n_kv].  A workgroup owns 256
// consecutive rows (4 waves x 64) and streams 128-key blocks of index_k through
// double-buffered LDS.  Each wave computes S^T = K * Q^T with the gfx950
// 32x32x16 bf16 MFMA, so that a lane's accumulators hold 16 keys of a single
// query column: the max-pool is in-lane plus one exchange between the two
// half-waves, and each lane ends every block with exactly one pooled value
// (its own row).  Products of bf16 values are exact in fp32; accumulation is
// fp32.  Causal masking (key j > p -> -inf) is applied only on blocks that
// reach past the wave's first position.
//
// FP8 index inputs (EB = 1; page "MiniMax lança MSA…", section "Kernel open
// source e MiniMax-M3": the released kernels take FP8 as well as BF16) run the
// same loop on the 32x32x64 E4M3 MFMA: half the bytes per key row, a quarter
// of the k-steps, the same accumulator layout and epilogue.
#include <type_traits>

#include "launch.h"

namespace msa {
namespace {

// EB: bytes per index element, 2 (bf16) or 1 (FP8 E4M3).
template <int DIDX, int EB>
struct IdxCfg {
  static constexpr bool F8 = EB == 1;
  static constexpr int ROWB = DIDX * EB;            // bytes per key row
  static constexpr int KB = F8 ? 64 : 16;           // index elements per MFMA k-step
  static constexpr int KS = DIDX / KB;              // MFMA k-steps per key row
  static constexpr int FB = F8 ? 32 : 16;           // operand bytes per lane per k-step
  static constexpr int RPK = F8 ? 4 : 2;            // 16-byte LDS reads per k-step (two key rows)
  static constexpr int CPR = ROWB / 16;             // 16-byte chunks per key row
  static constexpr int RPI = 1024 / ROWB;           // key rows per 1 KB direct-to-LDS instruction
  static constexpr int NG = kBk / RPI;              // such instructions per block
  static constexpr int NI = NG / 4;                 // per wave
  // LDS layout of a block.  Instruction g writes its 1 KB (RPI rows, row slot j
  // at j * ROWB, chunks in order) at g * PITCH; the 16-byte pad shifts each
  // instruction's rows by one bank group.  The rows an instruction holds are
  // chosen so that (a) a 32-key tile k (key rows 32k..32k+31) sits 256 k bytes
  // past tile 0 in every slot, so a lane's fragment address is one base plus an
  // immediate offset, and (b) the 16 lanes reading one chunk of rows
  // 32k+16h..32k+16h+15 land on 16 different bank groups:
  //   ROWB 256: row r in instruction r % 32, slot r / 32;
  //   ROWB 128: instruction r % 16, slot r / 16;
  //   ROWB  64: instruction r % 4 + 4 ((r / 16) % 2), slot (r / 4) % 4 + 4 (r / 32).
  static constexpr int PITCH = 1024 + 16;
  // byte offset, within the block's keys in HBM, of the chunk lane l of
  // instruction g fetches: dma_group(g) (uniform) + dma_lane(l)
  static __device__ __forceinline__ int dma_group(int g) {
    return ROWB == 256 ? 256 * g : ROWB == 128 ? 128 * g : 64 * (16 * (g / 4) + g % 4);
  }
  static __device__ __forceinline__ int dma_lane(int l) {
    const int j = l / CPR, c = l % CPR;
    return (ROWB == 256 ? 32 * 256 * j : ROWB == 128 ? 16 * 128 * j : 64 * (32 * (j / 4) + 4 * (j % 4))) + 16 * c;
  }
  // LDS byte offset of chunk 0 of key row r
  static __device__ __forceinline__ int lds_row(int r) {
    const int g = ROWB == 256 ? r % 32 : ROWB == 128 ? r % 16 : r % 4 + 4 * ((r / 16) % 2);
    const int j = ROWB == 256 ? r / 32 : ROWB == 128 ? r / 16 : (r / 4) % 4 + 4 * (r / 32);
    return g * PITCH + j * ROWB;
  }
  using Frag = std::conditional_t<F8, i32x8, uint4>;
};

// Sort the KK selected block ids of a lane ascending (bitonic network over a
// power-of-two padding; unused slots carry INT_MAX).
template <int KK>
__device__ __forceinline__ void sort_ids(int (&ti)[KK]) {
  constexpr int N = KK <= 8 ? 8 : 16;
  int x[N];
#pragma unroll
  for (int s = 0; s < N; ++s) x[s] = s < KK ? ti[s] : 0x7FFFFFFF;
#pragma unroll
  for (int size = 2; size <= N; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
#pragma unroll
      for (int s = 0; s < N; ++s) {
        const int o = s ^ stride;
        if (o > s) {
          const bool asc = (s & size) == 0;
          const int lo = min(x[s], x[o]), hi = max(x[s], x[o]);
          x[s] = asc ? lo : hi;
          x[o] = asc ? hi : lo;
        }
      }
    }
  }
#pragma unroll
  for (int s = 0; s < KK; ++s) ti[s] = x[s];
}

// KK == 0: write the pooled scores.  KK > 0: the launch covers every block of
// every row (no key split); each lane keeps its row's best KK non-local blocks
// by (score desc, index asc) in registers and writes the block_idx row (k = KK+1)
// exactly as the standalone top-k does from the same fp32 scores.
template <int DIDX, int KK, bool VL, int EB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_index_scores(
    const unsigned char* __restrict__ iq, const unsigned char* __restrict__ ik, float* __restrict__ pooled,
    int32_t* __restrict__ block_idx, Dims D, int32_t blocks_per_split) {
  using C = IdxCfg<DIDX, EB>;
  using Frag = typename C::Frag;
  // two key blocks (in the tile-interleaved layout of IdxCfg) as two separate arrays, each
  // named statically where it is used: the compiler can then tell a read of
  // one from the direct-to-LDS loads filling the other and does not wait for them
  __shared__ __align__(16) unsigned char lds0[C::NG * C::PITCH];
  __shared__ __align__(16) unsigned char lds1[C::NG * C::PITCH];
  __shared__ __align__(16) float pstage[KK == 0 ? 4 : 1][64][kPoolStage];  // per-lane pooled staging
  const float NEG_INF = -__builtin_huge_valf();

  const int b = blockIdx.z;
  const int rows_total = nq_of<VL>(D, b) * D.h_kv;    // this sequence's (query, group) rows
  const int64_t off_b = off_of<VL>(D, b);
  const int nkv_b = nkv_of<VL>(D, b);
  const int tile = gridDim.x - 1 - blockIdx.x;     // heaviest (latest) rows first
  const int row0 = tile * 256;
  if (VL && row0 >= rows_total) return;            // uniform over the workgroup
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int half = lane >> 5, col = lane & 31;

  const int last_row = min(row0 + 255, rows_total - 1);
  const int t_last = (int)((off_b + last_row / D.h_kv) / kBk);
  const int t_begin = blockIdx.y * blocks_per_split;
  const int t_end = min(t_begin + blocks_per_split, t_last + 1);
  if (t_begin >= t_end) return;  // uniform over the workgroup

  const int wrow0 = row0 + wave * 64;
  const bool wave_active = wrow0 < rows_total;
  const int64_t p_wave_min = off_b + (int64_t)(wave_active ? wrow0 : 0) / D.h_kv;

  // B operand: this lane's query columns (n-tile 0: row wrow0+col, n-tile 1: +32),
  // FB bytes of the index dim per k-step (8 bf16 or 32 E4M3 values).
  int64_t pc[2];
  Frag qb[2][C::KS];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int r = wrow0 + 32 * nt + col;
    if (r < rows_total) {
      pc[nt] = off_b + r / D.h_kv;
      const int64_t qr = VL ? qrow_of<VL>(D, b, r / D.h_kv) * D.h_kv + r % D.h_kv : (int64_t)b * rows_total + r;
      const unsigned char* src = iq + qr * C::ROWB + C::FB * half;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        if constexpr (C::F8)
          qb[nt][ks] = join32(*reinterpret_cast<const u32x4*>(src + 64 * ks),
                              *reinterpret_cast<const u32x4*>(src + 64 * ks + 16));
        else
          qb[nt][ks] = *reinterpret_cast<const uint4*>(src + 32 * ks);
      }
    } else {
      pc[nt] = -1;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) qb[nt][ks] = Frag{};
    }
  }

  // The row this lane owns: lane < 32 -> n-tile 0 column `lane`, else n-tile 1.
  const int r_out = wrow0 + lane;
  int64_t out_row = -1;  // (b, g, i) row index
  int l_out = -1;
  if (r_out < rows_total) {
    const int i = r_out / D.h_kv, g = r_out % D.h_kv;
    out_row = ((int64_t)b * D.h_kv + g) * D.n_q + i;
    l_out = (int)((off_b + i) / kBk);
  }
  float tv[KK > 0 ? KK : 1];
  int ti[KK > 0 ? KK : 1];
#pragma unroll
  for (int s = 0; s < (KK > 0 ? KK : 1); ++s) {
    tv[s] = NEG_INF;
    ti[s] = -1;
  }

  // KK > 0: a block whose score beats the lane's current KK-th waits in a
  // per-lane LDS list; the lists are merged into the registers, in block order,
  // once some lane's list is nearly full and at the end.  The wave then runs the
  // insertion once per few candidates of its busiest lane instead of in every
  // block where any of its 64 rows has one.  The merge tests each candidate
  // against the KK-th score of that moment, and the listing test admits a
  // superset of those, so the kept set is the one that inserting at every block
  // would keep.
  constexpr int kCand = 7;  // entries per lane: 4 waves x 7 x 64 x 8 bytes = 14 KB
  __shared__ float2 cand[KK > 0 ? 4 : 1][KK > 0 ? kCand : 1][64];
  int n_cand = 0;
  // insert (v, bt) into the lane's list sorted by (score desc, block asc); an
  // equal score never displaces an earlier block
  auto insert = [&](float v, int bt) {
    bool ge[KK > 0 ? KK : 1];
#pragma unroll
    for (int s = 0; s < KK; ++s) ge[s] = tv[s] >= v;
#pragma unroll
    for (int s = KK - 1; s >= 0; --s) {
      const bool here = s == 0 || ge[s - 1];
      const float sv = here ? v : tv[s > 0 ? s - 1 : 0];
      const int si = here ? bt : ti[s > 0 ? s - 1 : 0];
      tv[s] = ge[s] ? tv[s] : sv;
      ti[s] = ge[s] ? ti[s] : si;
    }
  };
  auto merge = [&]() {
#pragma unroll 1
    for (int j = 0; j < kCand; ++j) {
      if (j < n_cand) {
        const float2 e = cand[wave][j][lane];
        if (e.x > tv[KK > 0 ? KK - 1 : 0]) insert(e.x, __float_as_int(e.y));
      }
    }
    n_cand = 0;
  };

  // Key blocks arrive by direct buffer-to-LDS loads one block ahead, in the
  // layout above: the hardware writes lane l's 16 bytes at l * 16 past the
  // instruction's LDS address.  Each instruction gets a scalar descriptor whose
  // base is its uniform part of the block and whose record count stops at the
  // cache end: the range check drops the loads of keys past it, whose LDS rows
  // keep stale bytes that the causal mask replaces by -inf (a select, so any
  // bit pattern goes) before they are pooled, as those keys follow every row's
  // position.  The lane part of every load is one loop-invariant register.
  const unsigned char* ikb = ik + (int64_t)b * D.n_kv * C::ROWB;  // uniform case: sequence b's keys
  const uint32_t dma_off = C::dma_lane(lane);
  auto fetch_block = [&](int t, unsigned char* dst) {
    // the block's keys are contiguous (a page when paged); `n_cached` of them
    // (at least one) precede the cache end
    const unsigned char* blk;
    int n_cached;
    if constexpr (VL) {
      blk = ik + ikoff_of<VL>(D, b, t) * EB;
      n_cached = nkv_b - t * kBk;
    } else {
      blk = ikb + (int64_t)t * kBk * C::ROWB;
      n_cached = D.n_kv - t * kBk;
    }
    const int bytes = min(n_cached, kBk) * C::ROWB;
#pragma unroll
    for (int u = 0; u < C::NI; ++u) {
      const int g = wave * C::NI + u;
      const int go = C::dma_group(g);
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<unsigned char*>(blk) + go, (short)0, max(bytes - go, 0), kRawBufferFlags);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(dst + g * C::PITCH), 16,
                                               dma_off, 0, 0, 0);
    }
  };
  // this lane's fragment base: key row `col` (tile 0), its half's chunk
  const int rd_base = C::lds_row(col) + (C::F8 ? 32 : 16) * half;

  fetch_block(t_begin, lds0);
  auto process = [&](int t, auto buf_c) {
    constexpr int buf = decltype(buf_c)::value;
    const unsigned char* cur = buf == 0 ? lds0 : lds1;
    // this wave's part of block t has landed; after the barrier every part has,
    // and every wave is done with block t-1, whose buffer takes block t+1
    // (past the end: a repeat of the last block, never used, so that every
    // path issues the same loads)
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    fetch_block(min(t + 1, t_end - 1), buf == 0 ? lds1 : lds0);
    if (wave_active) {
      const bool need_mask = (int64_t)t * kBk + kBk - 1 > p_wave_min;
      float run0 = NEG_INF, run1 = NEG_INF;
      // this lane's FB bytes of k-step ks of its key row in tile k (chunk
      // 2ks+half, or chunks 4ks+2half and the next for E4M3): immediate offsets
      const unsigned char* rd = cur + rd_base;
      auto frag = [&](int k, int ks) -> Frag {
        const unsigned char* p = rd + 256 * k + C::FB * 2 * ks;
        if constexpr (C::F8)
          return join32(*reinterpret_cast<const u32x4*>(p), *reinterpret_cast<const u32x4*>(p + 16));
        else
          return *reinterpret_cast<const uint4*>(p);
      };
      auto mma = [&](Frag a, Frag bq, f32x16 c) {
        if constexpr (C::F8) return mfma_f8_32x32x64(a, bq, c);
        else return mfma_32x32x16(a, bq, c);
      };
      // max-pool of one 32-key tile's two query tiles: max(max(r, a), b) is one v_max3 per two scores
      auto pool_tile = [&](const f32x16& x0, const f32x16& x1) {
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
          run0 = fmaxf(fmaxf(run0, x0[e]), x0[e + 1]);
          run1 = fmaxf(fmaxf(run1, x1[e]), x1[e + 1]);
        }
      };
      if (!need_mask) {
        // Every key of the block is visible to every row of the wave.  The four
        // 32-key tiles form one straight-line region in which tile k's MFMAs
        // (two chains, each LDS fragment feeding both) are interleaved with the
        // max-pool of tile k-1, so the pool's VALU work issues while the MFMA
        // pipe is busy; only the last tile's pool is left after the MFMAs.
        // Software-pipelined over the 4 KS steps (tile k = st / KS, k-step
        // st % KS): step st's fragment is read two steps ahead into a ring of
        // three, and tile k-1's pool is spread over tile k's steps.  A
        // scheduling barrier closes each step, so the compiler cannot sink the
        // reads back next to their MFMAs to save registers.
        constexpr int STEPS = 4 * C::KS, EPS = 16 / C::KS;  // pooled elements per accumulator per step
        Frag fr[3];
        f32x16 acc[2][2];  // [tile parity][query tile]
        fr[0] = frag(0, 0);
        if (STEPS > 1) fr[1] = frag(1 / C::KS, 1 % C::KS);
#pragma unroll
        for (int st = 0; st < STEPS; ++st) {
          const int k = st / C::KS, ks = st % C::KS;
          if (st + 2 < STEPS) fr[(st + 2) % 3] = frag((st + 2) / C::KS, (st + 2) % C::KS);
          f32x16& x0 = acc[k & 1][0];
          f32x16& x1 = acc[k & 1][1];
          x0 = mma(fr[st % 3], qb[0][ks], ks == 0 ? f32x16{} : x0);
          x1 = mma(fr[st % 3], qb[1][ks], ks == 0 ? f32x16{} : x1);
          if (k > 0) {
            const f32x16& p0 = acc[(k - 1) & 1][0];
            const f32x16& p1 = acc[(k - 1) & 1][1];
#pragma unroll
            for (int e = EPS * ks; e < EPS * (ks + 1); e += 2) {  // max(max(r, a), b): one v_max3
              run0 = fmaxf(fmaxf(run0, p0[e]), p0[e + 1]);
              run1 = fmaxf(fmaxf(run1, p1[e]), p1[e + 1]);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        pool_tile(acc[1][0], acc[1][1]);
      } else {
        // two 32-key row tiles per iteration: four MFMA chains (32 bf16 or 8 E4M3
        // MFMAs) between epilogues, each LDS fragment feeding two MFMAs
#pragma unroll 1
        for (int mp = 0; mp < 2; ++mp) {
          f32x16 a00 = {}, a01 = {}, a10 = {}, a11 = {};
#pragma unroll
          for (int ks = 0; ks < C::KS; ++ks) {
            const Frag f0 = frag(2 * mp, ks);
            const Frag f1 = frag(2 * mp + 1, ks);
            a00 = mma(f0, qb[0][ks], a00);
            a01 = mma(f0, qb[1][ks], a01);
            a10 = mma(f1, qb[0][ks], a10);
            a11 = mma(f1, qb[1][ks], a11);
          }
          // LDS reads two k-steps ahead of their MFMAs
          constexpr int AHEAD = C::KS < 2 ? C::KS : 2;
          __builtin_amdgcn_sched_group_barrier(0x100, C::RPK * AHEAD, 0);
#pragma unroll
          for (int ks = 0; ks < C::KS; ++ks) {
            if (ks + 2 < C::KS) __builtin_amdgcn_sched_group_barrier(0x100, C::RPK, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
          }
          // key (t*Bk + 32*mt + row) is visible to column position p iff row <= p - (t*Bk + 32*mt)
          auto mask = [&](f32x16& x0, f32x16& x1, int mt) {
            const int64_t base = (int64_t)t * kBk + 32 * mt;
            const int rel0 = (int)max<int64_t>(-1, min<int64_t>(64, pc[0] - base)) - 4 * half;
            const int rel1 = (int)max<int64_t>(-1, min<int64_t>(64, pc[1] - base)) - 4 * half;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int row = 8 * (e >> 2) + (e & 3);
              if (row > rel0) x0[e] = NEG_INF;
              if (row > rel1) x1[e] = NEG_INF;
            }
          };
          mask(a00, a01, 2 * mp);
          mask(a10, a11, 2 * mp + 1);
          pool_tile(a00, a01);
          pool_tile(a10, a11);
        }
      }
      run0 = fmaxf(run0, wave_xor32(run0));
      run1 = fmaxf(run1, wave_xor32(run1));
      const float v = half ? run1 : run0;
      if constexpr (KK == 0) {
        // stage per lane; flush kPoolStage consecutive blocks of the row at once
        const int j = (t - t_begin) % kPoolStage;
        pstage[wave][lane][j] = v;
        if ((j == kPoolStage - 1 || t == t_end - 1) && out_row >= 0) {
          const int tb = t - j;
          const int n = min(j + 1, l_out - tb + 1);
          float* dst = pooled + out_row * D.n_blk + tb;
          if (n == kPoolStage && (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
            const float4* srcv = reinterpret_cast<const float4*>(&pstage[wave][lane][0]);
#pragma unroll
            for (int u = 0; u < kPoolStage / 4; ++u) reinterpret_cast<float4*>(dst)[u] = srcv[u];
          } else {
            for (int u = 0; u < n; ++u) dst[u] = pstage[wave][lane][u];
          }
        }
      } else {
        // a candidate for the running top-KK of the non-local blocks (t < l_out)
        if (t < l_out && v > tv[KK - 1]) {
          cand[wave][n_cand][lane] = make_float2(v, __int_as_float(t));
          ++n_cand;
        }
      }
    }
  };
  for (int t = t_begin; t < t_end; t += 2) {
    process(t, std::integral_constant<int, 0>{});
    if (t + 1 < t_end) process(t + 1, std::integral_constant<int, 1>{});
    // a pair of blocks lists at most two: merge while every list has room for them
    if constexpr (KK > 0)
      if (wave_active && __builtin_amdgcn_ballot_w64(n_cand > kCand - 2) != 0) merge();
  }
  if constexpr (KK > 0)
    if (wave_active) merge();
  __builtin_amdgcn_s_waitcnt(kWaitVm0);  // the last (unused) block fetch has landed before the workgroup ends

  if constexpr (KK > 0) {
    if (out_row >= 0) {
      int32_t* dst = block_idx + out_row * (KK + 1);
      if (l_out <= KK) {  // every visible block is kept
#pragma unroll
        for (int s = 0; s <= KK; ++s) dst[s] = s <= l_out ? s : -1;
      } else {
        sort_ids<KK>(ti);
#pragma unroll
        for (int s = 0; s < KK; ++s) dst[s] = ti[s];
        dst[KK] = l_out;
      }
    }
  }
}

}  // namespace

// Key-range splits so that row tiles x splits fill the chip (two workgroups per CU).
static int index_splits(const Dims& D, int row_tiles, int t_max, int* per) {
  const int64_t want = 512;
  int64_t nsplit = (want + (int64_t)row_tiles * D.B - 1) / ((int64_t)row_tiles * D.B);
  if (nsplit < 1) nsplit = 1;
  if (nsplit > t_max) nsplit = t_max;
  int p = (int)((t_max + nsplit - 1) / nsplit);
  p = (p + kPoolStage - 1) / kPoolStage * kPoolStage;  // splits start on a staging boundary
  *per = p;
  return (int)((t_max + p - 1) / p);
}

static void index_grid(const Dims& D, dim3* grid, int* per) {
  const int64_t rows_total = (int64_t)D.n_q * D.h_kv;
  const int row_tiles = (int)((rows_total + 255) / 256);
  const int t_max = (int)((D.offset + D.n_q - 1) / kBk) + 1;  // blocks the last row needs
  const int nsplit = index_splits(D, row_tiles, t_max, per);
  *grid = dim3(row_tiles, (unsigned)nsplit, D.B);
}

// Launch k_index_scores<DIDX, KK, VL, EB> for the runtime d_idx, batch kind and
// index element type.
template <int KK>
static void launch_index_kernel(const Dims& D, dim3 grid, int per, const void* index_q, const void* index_k,
                                float* pooled, int32_t* block_idx, hipStream_t stream) {
  auto iq = static_cast<const unsigned char*>(index_q);
  auto ik = static_cast<const unsigned char*>(index_k);
  auto go = [&](auto didx, auto vl, auto eb) {
    hipLaunchKernelGGL((k_index_scores<decltype(didx)::value, KK, decltype(vl)::value, decltype(eb)::value>), grid,
                       dim3(256), 0, stream, iq, ik, pooled, block_idx, D, per);
    mark(KK > 0 ? "k_index_scores(top-k fused)" : "k_index_scores", stream);
  };
  using I128 = std::integral_constant<int, 128>;
  using I64 = std::integral_constant<int, 64>;
  using T = std::true_type;
  using F = std::false_type;
  using E2 = std::integral_constant<int, 2>;
  using E1 = std::integral_constant<int, 1>;
  const bool vl = dims_varlen(D), f8 = D.idx_eb == 1;
  if (D.d_idx == 128) {
    if (f8) { if (vl) go(I128{}, T{}, E1{}); else go(I128{}, F{}, E1{}); }
    else    { if (vl) go(I128{}, T{}, E2{}); else go(I128{}, F{}, E2{}); }
  } else {
    if (f8) { if (vl) go(I64{}, T{}, E1{}); else go(I64{}, F{}, E1{}); }
    else    { if (vl) go(I64{}, T{}, E2{}); else go(I64{}, F{}, E2{}); }
  }
}

hipError_t launch_index_scores(const void* index_q, const void* index_k, float* pooled, const Dims& D,
                               hipStream_t stream) {
  dim3 grid;
  int per;
  index_grid(D, &grid, &per);
  launch_index_kernel<0>(D, grid, per, index_q, index_k, pooled, nullptr, stream);
  return hipGetLastError();
}

bool index_topk_fusable(const Dims& D) {
  if (D.k != 8 && D.k != 16) return false;
  dim3 grid;
  int per;
  index_grid(D, &grid, &per);
  return grid.y == 1;
}

hipError_t launch_index_topk(const void* index_q, const void* index_k, int32_t* block_idx, const Dims& D,
                             hipStream_t stream) {
  dim3 grid;
  int per;
  index_grid(D, &grid, &per);
  if (D.k == 16) launch_index_kernel<15>(D, grid, per, index_q, index_k, nullptr, block_idx, stream);
  else launch_index_kernel<7>(D, grid, per, index_q, index_k, nullptr, block_idx, stream);
  return hipGetLastError();
}

}  // namespace msa
