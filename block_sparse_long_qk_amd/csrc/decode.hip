// Decode-shaped calls: a few query rows per sequence against a long cache.
//
// Page "MiniMax 发布 MSA 稀疏注意力方法，开源推理内核并推出 MiniMax-M3 模型":
// section 两个分支如何工作 (index scores of the visible keys, max-pooled to
// blocks; softmax attention over the selected blocks) and section 优势与不足
// (decode at long context).  With one new token per sequence the index branch
// must stream every index key once: it is bound by HBM, not by the MFMA.
//
// k_index_small: (query, group) rows of one sequence (at most 16) form the
//   MFMA B operand in registers; every wave streams its own range of 128-key
//   blocks of index_k with coalesced loads into a register ring one block
//   deep, parks each 32-key step in a per-wave LDS buffer, reads it back as
//   16x16x32 bf16 MFMA A operands (no workgroup barriers) and max-pools each
//   block in registers.
// k_attn_rows: query-outer attention.  One wave per (row, slot): it loads the
//   slot's K block as MFMA B operands, computes the G x 128 scores, the block's
//   softmax statistics, and P V on the VALU from coalesced V rows; it writes an
//   fp32 partial and its base-2 log-sum-exp.
// k_merge_rows: LSE merge of a row's partials into bf16 out and the lse.
#include "launch.h"

namespace msa {
namespace {


__device__ __forceinline__ f32x4 mfma_16x16x32(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Each wave streams its own range of 128-key blocks in steps of 32 keys.  A
// step's 32 * DIDX * 2 bytes are read with fully coalesced 16-byte loads (64
// lanes cover one contiguous 1 KB span per instruction) into a register ring
// one block (four steps) deep, so 32 KB per wave are always in flight; each
// step is parked in the wave's LDS buffer (padded key rows), read back as
// 16x16x32 MFMA A operands (lane = key, lane group c = 8 index dims of each
// k-step) and max-pooled, and its ring slot is refilled with the same step of
// the next block.  Only wave-level ordering is needed: no workgroup barrier.
// Loads past the cache end repeat its last key (masked: it follows every
// row's position).  Pooled values wait in LDS and leave in batches, so stores
// rarely interrupt the load stream.  EB = 1 (FP8 E4M3 index inputs) uses the
// 16x16x128 E4M3 MFMA instead: lane group c supplies bytes [32c, 32c + 32) of
// a key and of a query row, one MFMA per 16 keys (index dim 64: groups 2 and 3
// supply zeros).
template <int DIDX, bool VL, int EB>
__global__ __launch_bounds__(256) void k_index_small(const unsigned char* __restrict__ iq,
                                                     const unsigned char* __restrict__ ik, float* __restrict__ pooled,
                                                     Dims D, int32_t blocks_per_wave) {
  constexpr bool F8 = EB == 1;
  constexpr int KS = F8 ? 1 : DIDX / 32;   // MFMA k-steps per key (16x16x32 bf16, 16x16x128 E4M3)
  constexpr int ROW = DIDX * EB;           // bytes per key
  constexpr int PITCH = ROW + 16;          // LDS bytes per key (pad: conflict-free operand reads)
  constexpr int STEP_KEYS = 32;
  constexpr int NSTEP = kBk / STEP_KEYS;   // steps per block = ring depth
  constexpr int LOADS = STEP_KEYS * ROW / 1024;  // 16-byte loads per lane per step
  constexpr int KEYS_PER_LOAD = 1024 / ROW;      // keys one load instruction covers
  constexpr int FLUSH = 16;                // pooled values staged per row before a store batch
  __shared__ __align__(16) unsigned char lds[4][STEP_KEYS * PITCH];
  __shared__ float pst[4][16][FLUSH];
  const float NEG_INF = -__builtin_huge_valf();
  const int b = blockIdx.y;
  const int nq_b = nq_of<VL>(D, b);
  if (nq_b == 0) return;          // uniform over the workgroup
  const int R = nq_b * D.h_kv;    // <= 16
  const int64_t off_b = off_of<VL>(D, b);
  const int nkv_b = nkv_of<VL>(D, b);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, c = lane >> 4;
  const int t_last = (int)((off_b + nq_b - 1) / kBk);
  const int t0 = ((int)blockIdx.x * 4 + wave) * blocks_per_wave;
  const int t1 = min(t0 + blocks_per_wave, t_last + 1);
  if (t0 >= t1) return;

  using Frag = std::conditional_t<F8, i32x8, uint4>;
  Frag qb[KS];
  const bool row_ok = n < R;
  const int64_t pc = row_ok ? off_b + n / D.h_kv : -1;
  const int l_row = row_ok ? (int)(pc / kBk) : -1;
  // E4M3 with index dim 64: lane groups 2 and 3 hold no index dims
  const bool c_ok = !F8 || 32 * c < ROW;
  {
    const unsigned char* qrow =
        iq + (row_ok ? (qrow_of<VL>(D, b, n / D.h_kv) * D.h_kv + n % D.h_kv) * ROW : 0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if constexpr (F8)
        qb[ks] = row_ok && c_ok ? join32(*reinterpret_cast<const u32x4*>(qrow + 32 * c),
                                         *reinterpret_cast<const u32x4*>(qrow + 32 * c + 16))
                                : i32x8{};
      else
        qb[ks] = row_ok ? *reinterpret_cast<const uint4*>(qrow + 16 * (KS * c + ks)) : make_uint4(0, 0, 0, 0);
    }
  }
  int64_t out_base = -1;
  if (row_ok) {
    const int i = n / D.h_kv, g = n % D.h_kv;
    out_base = (((int64_t)b * D.h_kv + g) * D.n_q + i) * D.n_blk;
  }
  unsigned char* buf = lds[wave];
  // this lane's slot in a load: key u*KEYS_PER_LOAD + lk, byte offset lo
  const int lk = (lane * 16) / ROW, lo = (lane * 16) % ROW;
  auto fetch = [&](int t, int st, u32x4 (&x)[LOADS]) {
    // the block's keys are contiguous (a page when paged); past the cache end
    // its last key repeats
    const unsigned char* blk = ik + ikoff_of<VL>(D, b, t) * EB;
    const int last = nkv_b - 1 - t * kBk;
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int key = min(st * STEP_KEYS + u * KEYS_PER_LOAD + lk, last);
      x[u] = *reinterpret_cast<const u32x4*>(blk + key * ROW + lo);
    }
  };
  u32x4 ring[NSTEP][LOADS];  // native vectors: whole-register copies, no memcpy
#pragma unroll
  for (int st = 0; st < NSTEP; ++st) {  // in slot order, as the loop refills them
    fetch(t0, st, ring[st]);
    __builtin_amdgcn_sched_barrier(0);
  }

  auto flush = [&](int tb, int cnt) {
    if (c == 0 && out_base >= 0) {
      for (int j = 0; j < cnt; ++j)
        if (tb + j <= l_row) pooled[out_base + tb + j] = pst[wave][n][j];
    }
  };
  int tb = t0;
  for (int t = t0; t < t1; ++t) {
    const int tn = min(t + 1, t1 - 1);  // next block (past the end: a repeat, never used)
    float m = NEG_INF;
#pragma unroll
    for (int st = 0; st < NSTEP; ++st) {
      // park step st, refill its slot with the next block's step st
#pragma unroll
      for (int u = 0; u < LOADS; ++u)
        *reinterpret_cast<u32x4*>(buf + (u * KEYS_PER_LOAD + lk) * PITCH + lo) = ring[st][u];
      __builtin_amdgcn_sched_barrier(0);
      fetch(tn, st, ring[st]);
      __builtin_amdgcn_sched_barrier(0);
      wave_lds_fence();
      const int64_t skey0 = (int64_t)t * kBk + st * STEP_KEYS;
      const bool need_mask = skey0 + STEP_KEYS - 1 > off_b;
#pragma unroll
      for (int T = 0; T < STEP_KEYS / 16; ++T) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        const unsigned char* krow = buf + (16 * T + n) * PITCH;
        if constexpr (F8) {
          const i32x8 a = c_ok ? join32(*reinterpret_cast<const u32x4*>(krow + 32 * c),
                                        *reinterpret_cast<const u32x4*>(krow + 32 * c + 16))
                               : i32x8{};
          acc = mfma_f8_16x16x128(a, qb[0], acc);
        } else {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const uint4 a = *reinterpret_cast<const uint4*>(krow + 16 * (KS * c + ks));
            acc = mfma_16x16x32(a, qb[ks], acc);
          }
        }
        // accumulator j of lane (n, c) is key skey0 + 16*T + 4*c + j against row n
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float x = acc[j];
          if (need_mask && skey0 + 16 * T + 4 * c + j > pc) x = NEG_INF;
          m = fmaxf(m, x);
        }
      }
      wave_lds_fence();  // the buffer is rewritten next step
    }
    m = fmaxf(m, __shfl_xor(m, 16, 64));
    m = fmaxf(m, __shfl_xor(m, 32, 64));
    if (c == 0) pst[wave][n][t - tb] = m;
    if (t - tb == FLUSH - 1) {
      flush(tb, FLUSH);
      tb = t + 1;
    }
  }
  if (t1 > tb) flush(tb, t1 - tb);
}

// Is slot s of a row a block to attend?  Slot k stands for the local block
// when the row does not list it.
__device__ __forceinline__ int slot_block(const int32_t* row, int s, int k, int local) {
  if (s == k) {
    for (int u = 0; u < k; ++u)
      if (row[u] == local) return -1;
    return local;
  }
  const int t = row[s];
  return (t >= 0 && t <= local && (s == 0 || row[s - 1] != t)) ? t : -1;
}

// One wave per (row, slot); GMAX (8 or 16) >= G query heads of the row's group.
// KV8: K and V hold FP8 E4M3 codes (1 byte per element), widened to bf16 as
// they are loaded; the arithmetic is then the bf16 path's.
template <int GMAX, bool VL, bool KV8>
__global__ __launch_bounds__(256) void k_attn_rows(const uint16_t* __restrict__ q, const void* __restrict__ k,
                                                   const void* __restrict__ v,
                                                   const int32_t* __restrict__ block_idx, float* __restrict__ part,
                                                   Dims D) {
  __shared__ float P[4][kBk][GMAX];  // per wave: probabilities [key][head]
  __shared__ __align__(16) unsigned char Kst[4][32 * (kHeadDim * 2 + 16)];  // per wave: one 32-key step of K
  const float NEG_INF = -__builtin_huge_valf();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t r = blockIdx.x;  // row = (b*h_kv + g)*n_q + i
  const int s = blockIdx.y * 4 + wave;
  if (s > D.k) return;  // slots 0..k (k = the unlisted local block)
  const int64_t bg = r / D.n_q;
  const int i = (int)(r % D.n_q);
  const int g = (int)(bg % D.h_kv), b = (int)(bg / D.h_kv);
  if (i >= nq_of<VL>(D, b)) return;  // a row past this sequence's queries (whole workgroup)
  const int nkv_b = nkv_of<VL>(D, b);
  const int64_t p = off_of<VL>(D, b) + i;
  const int local = (int)(p / kBk);
  const int t = slot_block(block_idx + r * D.k, s, D.k, local);  // same for the whole wave
  float* dst = part + (r * (D.k + 1) + s) * (int64_t)kRowsPart;  // o [16][d], then lse [16]
  if (t < 0) {
    if (lane < 16) dst[16 * kHeadDim + lane] = NEG_INF;
    return;
  }
  const int n = lane & 15, c = lane >> 4;
  const int64_t key0 = (int64_t)t * kBk;
  constexpr int EBKV = KV8 ? 1 : 2;  // bytes per K/V element
  const unsigned char* kbytes = static_cast<const unsigned char*>(k) + kvoff_of<VL>(D, b, g, t) * EBKV;
  const unsigned char* vbytes = static_cast<const unsigned char*>(v) + kvoff_of<VL>(D, b, g, t) * EBKV;

  // scores S[h][key] with MFMA: A = Q (rows = heads), B = K^T (columns = keys);
  // lane group c and k-step ks hold head dims 32*c + 8*ks .. +8.
  uint4 qa[4];
  const bool head_ok = n < D.G;
  const uint16_t* qrow = q + (qrow_of<VL>(D, b, i) * D.h_q + g * D.G + (head_ok ? n : 0)) * kHeadDim + 32 * c;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    qa[ks] = head_ok ? *reinterpret_cast<const uint4*>(qrow + 8 * ks) : make_uint4(0, 0, 0, 0);
  // K in four 32-key steps: fully coalesced 16-byte loads (4 keys per
  // instruction) parked in this wave's padded LDS buffer, read back as MFMA B
  // operands; the next step's loads are in flight while this one computes.
  constexpr int KPITCH = kHeadDim * 2 + 16;  // bytes per key row in LDS
  unsigned char* kbuf = Kst[wave];
  const int lk = lane >> 4, lo = (lane & 15) * 16;
  const int n_keys = (int)min((int64_t)kBk, (int64_t)nkv_b - key0);
  uint4 kx[8];
  auto fetch_k = [&](int st) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int key = 32 * st + 4 * u + lk;
      if constexpr (KV8) {
        const uint2 c8 = key < n_keys ? *reinterpret_cast<const uint2*>(kbytes + key * kHeadDim + lo / 2)
                                      : make_uint2(0, 0);
        const u32x4 wv = e4m3x8_to_bf16(c8);
        kx[u] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
      } else {
        kx[u] = key < n_keys ? *reinterpret_cast<const uint4*>(kbytes + key * (kHeadDim * 2) + lo)
                             : make_uint4(0, 0, 0, 0);
      }
    }
  };
  f32x4 sc[8];
  fetch_k(0);
#pragma unroll
  for (int st = 0; st < 4; ++st) {
#pragma unroll
    for (int u = 0; u < 8; ++u) *reinterpret_cast<uint4*>(kbuf + (4 * u + lk) * KPITCH + lo) = kx[u];
    wave_lds_fence();
    if (st + 1 < 4) fetch_k(st + 1);
#pragma unroll
    for (int T2 = 0; T2 < 2; ++T2) {
      const int T = 2 * st + T2;
      sc[T] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const uint4 kf = *reinterpret_cast<const uint4*>(kbuf + (16 * T2 + n) * KPITCH + 16 * (4 * c + ks));
        sc[T] = mfma_16x16x32(qa[ks], kf, sc[T]);
      }
    }
    wave_lds_fence();
  }
  // lane (column key = 16T + n, group c) holds heads 4c + j; keys past p or n_kv drop
  float mx[4], sm[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float m = NEG_INF;
#pragma unroll
    for (int T = 0; T < 8; ++T) {
      const int64_t key = key0 + 16 * T + n;
      float x = sc[T][j] * D.scale_log2;
      if (key > p || key >= nkv_b) x = NEG_INF;
      sc[T][j] = x;
      m = fmaxf(m, x);
    }
    m = row16_reduce(m, [](float a, float b) { return fmaxf(a, b); });
    const float mref = m == NEG_INF ? 0.f : m;
    float sum = 0.f;
#pragma unroll
    for (int T = 0; T < 8; ++T) {
      const float e = __builtin_amdgcn_exp2f(sc[T][j] - mref);
      sum += e;
      if (4 * c + j < GMAX) P[wave][16 * T + n][4 * c + j] = e;
    }
    sum = row16_reduce(sum, [](float a, float b) { return a + b; });
    mx[j] = m;
    sm[j] = sum;
  }
  // per-head statistics to every lane (head h lives in lane group h / 4, register h % 4)
  float lh[GMAX], mh[GMAX];
#pragma unroll
  for (int h = 0; h < GMAX; ++h) {
    lh[h] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sm[h & 3]), 16 * (h >> 2)));
    mh[h] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mx[h & 3]), 16 * (h >> 2)));
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // O[h][8*dc .. +8] over keys kr, kr+4, ...: lane = (dc = lane % 16, kr = lane / 16)
  const int dc = lane & 15, kr = lane >> 4;
  float acc[GMAX][8];
#pragma unroll
  for (int h = 0; h < GMAX; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  // rows kr, kr+4, ...: eight rows' loads issued before their FMAs
#pragma unroll 1
  for (int kb8 = 0; kb8 < kBk; kb8 += 32) {
    uint4 w8[8];
    uint2 c8[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int kk = kb8 + 4 * u + kr;
      if constexpr (KV8)
        c8[u] = kk < n_keys ? *reinterpret_cast<const uint2*>(vbytes + kk * kHeadDim + 8 * dc) : make_uint2(0, 0);
      else
        w8[u] = kk < n_keys ? *reinterpret_cast<const uint4*>(vbytes + kk * (kHeadDim * 2) + 16 * dc)
                            : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int kk = kb8 + 4 * u + kr;
      if constexpr (KV8) {
        const u32x4 wv = e4m3x8_to_bf16(c8[u]);
        w8[u] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
      }
      const uint32_t x[4] = {w8[u].x, w8[u].y, w8[u].z, w8[u].w};
      float vv[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vv[2 * e] = __uint_as_float(x[e] << 16);
        vv[2 * e + 1] = __uint_as_float(x[e] & 0xFFFF0000u);
      }
#pragma unroll
      for (int h = 0; h < GMAX; ++h) {
        const float ph = P[wave][kk][h];  // zero past n_keys
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] += ph * vv[e];
      }
    }
  }
#pragma unroll
  for (int h = 0; h < GMAX; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = acc[h][e];
      x += __shfl_xor(x, 16, 64);
      x += __shfl_xor(x, 32, 64);
      acc[h][e] = x;
    }
  if (kr == 0) {
#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
      if (h < D.G) {
        const float inv = 1.f / lh[h];
        float4* o4 = reinterpret_cast<float4*>(dst + h * kHeadDim + 8 * dc);
        o4[0] = make_float4(acc[h][0] * inv, acc[h][1] * inv, acc[h][2] * inv, acc[h][3] * inv);
        o4[1] = make_float4(acc[h][4] * inv, acc[h][5] * inv, acc[h][6] * inv, acc[h][7] * inv);
      }
    }
  }
#pragma unroll
  for (int h = 0; h < GMAX; ++h)
    if (lane == h && h < D.G) dst[16 * kHeadDim + h] = mh[h] + __log2f(lh[h]);
}

// One workgroup per row: out[b][i][g*G + h][d] and lse from the row's partials.
template <bool VL>
__global__ __launch_bounds__(256) void k_merge_rows(const float* __restrict__ part, uint16_t* __restrict__ out,
                                                    float* __restrict__ lse_out, Dims D) {
  const float NEG_INF = -__builtin_huge_valf();
  const int64_t r = blockIdx.x;
  const int64_t bg = r / D.n_q;
  const int i = (int)(r % D.n_q);
  const int g = (int)(bg % D.h_kv), b = (int)(bg / D.h_kv);
  if (i >= nq_of<VL>(D, b)) return;  // a row past this sequence's queries (whole workgroup)
  const int nslot = D.k + 1;
  const float* base = part + r * nslot * (int64_t)kRowsPart;
  for (int x = threadIdx.x; x < D.G * (kHeadDim / 4); x += blockDim.x) {
    const int h = x / (kHeadDim / 4), d4 = x % (kHeadDim / 4);
    float m = NEG_INF;
    for (int s = 0; s < nslot; ++s) m = fmaxf(m, base[s * kRowsPart + 16 * kHeadDim + h]);
    float wsum = 0.f;
    for (int s = 0; s < nslot; ++s) {
      const float ls = base[s * kRowsPart + 16 * kHeadDim + h];
      if (ls > NEG_INF) wsum += __builtin_amdgcn_exp2f(ls - m);
    }
    const float tot = m + __log2f(wsum);
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = 0; s < nslot; ++s) {
      const float* ps = base + s * kRowsPart;
      const float ls = ps[16 * kHeadDim + h];
      if (!(ls > NEG_INF)) continue;
      const float cw = __builtin_amdgcn_exp2f(ls - tot);
      const float4 w = *reinterpret_cast<const float4*>(ps + h * kHeadDim + 4 * d4);
      o.x += cw * w.x;
      o.y += cw * w.y;
      o.z += cw * w.z;
      o.w += cw * w.w;
    }
    uint16_t* dst = out + (qrow_of<VL>(D, b, i) * D.h_q + g * D.G + h) * kHeadDim + 4 * d4;
    *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(o.x, o.y), pack_bf16x2(o.z, o.w));
    if (lse_out && d4 == 0) lse_out[((int64_t)b * D.h_q + g * D.G + h) * D.n_q + i] = tot * 0.69314718055994531f;
  }
}

}  // namespace

bool use_index_small(const Dims& D) { return (int64_t)D.n_q * D.h_kv <= 16; }

bool use_attn_rows(const Dims& D) { return D.n_q <= kRowsMaxQ && D.G <= 16; }

size_t attn_rows_partial_bytes(const Dims& D) {
  return sizeof(float) * (size_t)D.B * D.h_kv * D.n_q * (D.k + 1) * kRowsPart;
}

hipError_t launch_index_small(const void* index_q, const void* index_k, float* pooled, const Dims& D,
                              hipStream_t stream) {
  const int t_max = (int)((D.offset + D.n_q - 1) / kBk) + 1;
  // one resident round of waves over the whole batch (8 waves per CU: the
  // kernel holds two waves per SIMD), at least one block per wave, so every
  // wave fills its load ring once and then streams a long range
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu <= 0)
      ncu = 256;
    cus = ncu;
  }
  int64_t waves_per_b = (8LL * cus + D.B - 1) / D.B;
  if (waves_per_b > t_max) waves_per_b = t_max;
  const int per = (int)((t_max + waves_per_b - 1) / waves_per_b);
  const int wgs = (int)(((t_max + per - 1) / per + 3) / 4);
  dim3 grid(wgs, D.B);
  auto iq = static_cast<const unsigned char*>(index_q);
  auto ik = static_cast<const unsigned char*>(index_k);
  auto go = [&](auto didx, auto vl, auto eb) {
    hipLaunchKernelGGL((k_index_small<decltype(didx)::value, decltype(vl)::value, decltype(eb)::value>), grid,
                       dim3(256), 0, stream, iq, ik, pooled, D, per);
    mark("k_index_small", stream);
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
  return hipGetLastError();
}

hipError_t launch_attn_rows(const uint16_t* q, const void* k, const void* v, const int32_t* block_idx,
                            uint16_t* out, float* lse, float* part, const Dims& D, hipStream_t stream) {
  const int64_t rows = (int64_t)D.B * D.h_kv * D.n_q;
  dim3 grid((unsigned)rows, (D.k + 1 + 3) / 4);
  auto go = [&](auto gm, auto vlc, auto kv8) {
    hipLaunchKernelGGL((k_attn_rows<decltype(gm)::value, decltype(vlc)::value, decltype(kv8)::value>), grid,
                       dim3(256), 0, stream, q, k, v, block_idx, part, D);
    mark("k_attn_rows", stream);
  };
  auto by_kv = [&](auto gm, auto vlc) {
    if (D.kv_eb == 1) go(gm, vlc, std::true_type{}); else go(gm, vlc, std::false_type{});
  };
  auto by_vl = [&](auto gm) {
    if (dims_varlen(D)) by_kv(gm, std::true_type{}); else by_kv(gm, std::false_type{});
  };
  if (D.G <= 8) by_vl(std::integral_constant<int, 8>{}); else by_vl(std::integral_constant<int, 16>{});
  const bool vl = dims_varlen(D);
  if (vl)
    hipLaunchKernelGGL(k_merge_rows<true>, dim3((unsigned)rows), dim3(256), 0, stream, part, out, lse, D);
  else
    hipLaunchKernelGGL(k_merge_rows<false>, dim3((unsigned)rows), dim3(256), 0, stream, part, out, lse, D);
  mark("k_merge_rows", stream);
  return hipGetLastError();
}

}  // namespace msa
