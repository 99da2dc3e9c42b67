// Dense causal GQA attention: the Main Branch over every visible token, the
// mode both branches run in during the indexer warmup (page "MiniMax 发布 MSA
// 稀疏注意力方法，开源推理内核并推出 MiniMax-M3 模型", section MSA 如何训练: in the
// first iterations both branches run full attention, so that the indexer
// learns from the KL loss before it routes; page "MiniMax lança MSA…", item
// "Indexer Warmup").
//
// Query-outer with the KV stream through LDS (for dense attention every tile
// reads the same blocks 0 .. its own, so there is nothing to gather): a
// workgroup of 8 waves owns a tile of pt consecutive positions (aligned to pt,
// pt * G <= 256 rows, pt <= 128, so a tile never straddles a block) of one
// (sequence, group); each wave owns 32 rows.
// Per 128-key block: S^T = K Q^T and O^T += V^T P^T on 32x32x16 bf16 MFMA with
// an online softmax in base 2.  The query rows sit in each wave's LDS region
// (fetched once); block t+1's K and V are loaded into registers while block t
// is computed and written to LDS (V transposed) between two barriers.  Tiles are
// dealt heaviest first, and workgroup w of a (sequence, group) count B * h_kv
// divisible by 8 keeps one group per XCD (w % 8), so the tiles that stream a
// group's blocks share an L2.
#include "attn_tiles.h"

namespace msa {
namespace {

// One block of K and V in flight through registers: the loads of stage_kv,
// with the LDS writes split off so that they can follow the next compute
// (native vectors: whole-register copies, so the struct stays in registers).
struct KvRegs {
  u32x4 kr[2048 / kThreads];
  u32x4 vr[4 * (512 / kThreads)];
};

// V unit c (0 .. 511): key quad kq (keys 4kq .. 4kq+3) and 16-byte dim chunk od
// (dims 8od .. 8od+7).  A wave covers 8 key quads x 8 dim chunks, so that the
// 32 lanes of each half-wave write their transposed words (row 8od + e of V^T,
// keys 4kq ..) to 32 different bank pairs: with the rows 66 words apart, two
// chunks 4 apart meet in a bank, and 16 chunks x 2 quads per half-wave met
// four times in each.
__device__ __forceinline__ void v_unit(int c, int& kq, int& od) {
  const int w = c >> 6, l = c & 63;
  kq = 8 * (w & 3) + (l & 7);
  od = 8 * (w >> 2) + (l >> 3);
}

__device__ __forceinline__ void kv_load(KvRegs& x, const uint16_t* __restrict__ kb, const uint16_t* __restrict__ vb,
                                        int n_valid) {
  constexpr int KPER = 2048 / kThreads, VPER = 512 / kThreads;
  const int tid = threadIdx.x;
  const char* kbase = reinterpret_cast<const char*>(kb);
  const char* vbase = reinterpret_cast<const char*>(vb);
#pragma unroll
  for (int u = 0; u < KPER; ++u) {
    const int c = tid + kThreads * u;
    const uint32_t off = (uint32_t)min(c >> 4, n_valid - 1) * 256u + 16u * (c & 15);
    x.kr[u] = *reinterpret_cast<const u32x4*>(kbase + off);
  }
#pragma unroll
  for (int u = 0; u < VPER; ++u) {
    const int c = tid + kThreads * u;
    int kq, od;
    v_unit(c, kq, od);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t off = (uint32_t)min(kq * 4 + q, n_valid - 1) * 256u + 16u * od;
      x.vr[4 * u + q] = *reinterpret_cast<const u32x4*>(vbase + off);
    }
  }
}

__device__ __forceinline__ void kv_store(uint16_t* Ks, uint16_t* Vt, const KvRegs& x) {
  constexpr int KPER = 2048 / kThreads, VPER = 512 / kThreads;
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < KPER; ++u) {
    const int c = tid + kThreads * u;
    *reinterpret_cast<u32x4*>(Ks + (c >> 4) * KP + (c & 15) * 8) = x.kr[u];
  }
#pragma unroll
  for (int u = 0; u < VPER; ++u) {  // transposed: Vt[d][key]
    const int c = tid + kThreads * u;
    int kq, od;
    v_unit(c, kq, od);
    uint32_t w[4][4];  // by value: words of the four keys' 16-byte chunks
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4 y = x.vr[4 * u + q];
      w[q][0] = y.x;
      w[q][1] = y.y;
      w[q][2] = y.z;
      w[q][3] = y.w;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int sh = (e & 1) * 16;
      const uint32_t v0 = (w[0][e >> 1] >> sh) & 0xFFFFu, v1 = (w[1][e >> 1] >> sh) & 0xFFFFu;
      const uint32_t v2 = (w[2][e >> 1] >> sh) & 0xFFFFu, v3 = (w[3][e >> 1] >> sh) & 0xFFFFu;
      *reinterpret_cast<uint2*>(Vt + (od * 8 + e) * VP + kq * 4) = make_uint2(v0 | (v1 << 16), v2 | (v3 << 16));
    }
  }
}

// Dense tiles per (sequence, group): pt-aligned runs of positions covering the
// query positions.
__host__ __device__ __forceinline__ int dense_tiles(const Dims& D) {
  return (int)((D.offset + D.n_q - 1) / D.pt - D.offset / D.pt + 1);
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_dense_attn(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ out, float* __restrict__ lse_out, Dims D) {
  __shared__ __align__(16) uint16_t Ks[kBk * KP];
  __shared__ __align__(16) uint16_t Vt[kHeadDim * VP];
  __shared__ __align__(16) unsigned char Qs[kWaves][kQRegion];
  const float NEG_INF = -__builtin_huge_valf();

  const int nbg = D.B * D.h_kv, n_t = dense_tiles(D);
  const int bg = blockIdx.x % nbg;
  const int tile = n_t - 1 - (int)(blockIdx.x / nbg);   // heaviest first
  const int b = bg / D.h_kv, g = bg % D.h_kv;
  const int p0 = (int)((D.offset / D.pt + tile) * D.pt);  // first position (positions fit in 32 bits)
  const int t_last = p0 / kBk;                            // the block of every position of the tile

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 31, half = lane >> 5;
  const int r = wave * 32 + col;
  const int ps = r / D.G, hh = r % D.G;
  const int p = p0 + ps;
  const bool valid = ps < D.pt && p >= D.offset && p < D.offset + D.n_q;
  const int i = valid ? (int)(p - D.offset) : 0;
  unsigned char* qw = Qs[wave];

  const uint16_t* kg = k + ((int64_t)b * D.h_kv + g) * D.n_kv * kHeadDim;
  const uint16_t* vg = v + ((int64_t)b * D.h_kv + g) * D.n_kv * kHeadDim;
  auto n_valid = [&](int t) { return max(1, min(kBk, D.n_kv - t * kBk)); };

  // prologue: the query rows and block 0
  fetch_q_rows(qw, q + (((int64_t)b * D.n_q + i) * D.h_q + g * D.G + hh) * kHeadDim, lane);
  {
    KvRegs x;
    kv_load(x, kg, vg, n_valid(0));
    kv_store(Ks, Vt, x);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);  // this wave's query rows have landed
    __syncthreads();
  }

  f32x16 o[4];
#pragma unroll
  for (int d4 = 0; d4 < 4; ++d4) o[d4] = f32x16{};
  float m_run = NEG_INF, l_run = 0.f;  // l_run: this lane's share of the row sum
  const float c = D.scale_log2;
  for (int t = 0; t <= t_last; ++t) {
    const bool more = t < t_last;
    KvRegs x;
    if (more) kv_load(x, kg + (int64_t)(t + 1) * kBk * kHeadDim, vg + (int64_t)(t + 1) * kBk * kHeadDim, n_valid(t + 1));
    f32x16 s[4];
    __builtin_amdgcn_sched_barrier(0);
    qk_block(Ks, qw, lane, s);
    __builtin_amdgcn_sched_barrier(0);
    // online softmax in base 2; the last block (the diagonal) masks keys after the row's position
    const bool masked = t == t_last;
#pragma unroll
    for (int T = 0; T < 4; ++T) {
#pragma unroll
      for (int e = 0; e < 16; ++e) s[T][e] *= c;
    }
    if (masked) {  // uniform, and a branch of its own: the blocks before the diagonal skip it
      const int rel = max(-1, min(kBk, p - t * kBk)) - 4 * half;
#pragma unroll
      for (int T = 0; T < 4; ++T) {
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (32 * T + 8 * (e >> 2) + (e & 3) > rel) s[T][e] = NEG_INF;
      }
    }
    float mx = NEG_INF;
#pragma unroll
    for (int T = 0; T < 4; ++T) {
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[T][e]);
    }
    mx = fmaxf(mx, wave_xor32(mx));
    const float m_new = fmaxf(m_run, mx);
    const float mref = m_new == NEG_INF ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - mref);  // 0 on the first block
#pragma unroll
    for (int d4 = 0; d4 < 4; ++d4) {
#pragma unroll
      for (int e = 0; e < 16; ++e) o[d4][e] *= alpha;
    }
    l_run *= alpha;
    m_run = m_new;
#pragma unroll
    for (int T = 0; T < 4; ++T) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        s[T][e] = __builtin_amdgcn_exp2f(s[T][e] - mref);
        l_run += s[T][e];
      }
    }
    // O^T += V^T P^T (V operands of k-step j+1 read while step j runs).  On the
    // diagonal block, where a row's weight can sit on a few keys, each
    // probability enters as two bf16 parts, hi and lo = P - hi.
    const uint16_t* vbase = Vt + col * VP + 4 * half;
    auto read_v = [&](int j, uint4 (&dst)[4]) {
#pragma unroll
      for (int d4 = 0; d4 < 4; ++d4) {
        const uint16_t* vrow = vbase + 32 * d4 * VP + 16 * j;
        const uint2 lo = *reinterpret_cast<const uint2*>(vrow);
        const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 8);
        dst[d4] = make_uint4(lo.x, lo.y, hi.x, hi.y);
      }
    };
    uint4 vf[2][4];
    read_v(0, vf[0]);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int T = j >> 1, u = j & 1;
      if (j + 1 < 8) read_v(j + 1, vf[(j + 1) & 1]);
      uint32_t ph[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) ph[w] = pack_bf16x2(s[T][8 * u + 2 * w], s[T][8 * u + 2 * w + 1]);
      const uint4 pb = make_uint4(ph[0], ph[1], ph[2], ph[3]);
#pragma unroll
      for (int d4 = 0; d4 < 4; ++d4) o[d4] = mfma_32x32x16(vf[j & 1][d4], pb, o[d4]);
      if (masked) {
        uint32_t pl[4];
#pragma unroll
        for (int w = 0; w < 4; ++w)
          pl[w] = pack_bf16x2(s[T][8 * u + 2 * w] - __uint_as_float(ph[w] << 16),
                              s[T][8 * u + 2 * w + 1] - __uint_as_float(ph[w] & 0xFFFF0000u));
        const uint4 plo = make_uint4(pl[0], pl[1], pl[2], pl[3]);
#pragma unroll
        for (int d4 = 0; d4 < 4; ++d4) o[d4] = mfma_32x32x16(vf[j & 1][d4], plo, o[d4]);
      }
    }
    __syncthreads();  // every wave is done with block t
    if (more) {
      kv_store(Ks, Vt, x);
      __syncthreads();
    }
  }

  const float l = l_run + wave_xor32(l_run);
  if (valid) {
    const float inv = 1.f / l;
    // accumulator (d4, e) of lane (col, half) is head dim 32 d4 + 8 (e/4) + 4 half + e%4
    uint16_t* dst = out + (((int64_t)b * D.n_q + i) * D.h_q + g * D.G + hh) * kHeadDim + 4 * half;
#pragma unroll
    for (int d4 = 0; d4 < 4; ++d4) {
#pragma unroll
      for (int a = 0; a < 4; ++a)
        *reinterpret_cast<uint2*>(dst + 32 * d4 + 8 * a) =
            make_uint2(pack_bf16x2(o[d4][4 * a] * inv, o[d4][4 * a + 1] * inv),
                       pack_bf16x2(o[d4][4 * a + 2] * inv, o[d4][4 * a + 3] * inv));
    }
    if (lse_out && half == 0)
      lse_out[((int64_t)b * D.h_q + g * D.G + hh) * D.n_q + i] = (m_run + __log2f(l)) * 0.69314718055994531f;
  }
}

}  // namespace

int64_t dense_grid(const Dims& D) { return (int64_t)D.B * D.h_kv * dense_tiles(D); }

hipError_t launch_dense_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* out, float* lse,
                             const Dims& D, hipStream_t stream) {
  hipLaunchKernelGGL(k_dense_attn, dim3((unsigned)dense_grid(D)), dim3(kThreads), 0, stream, q, k, v, out, lse, D);
  return hipGetLastError();
}

}  // namespace msa
