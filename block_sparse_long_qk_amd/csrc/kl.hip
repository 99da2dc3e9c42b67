// KL alignment of the Index Branch to the Main Branch (the forward value of the
// loss that trains the index projections).
//
// Page "MiniMax 发布 MSA 稀疏注意力方法，开源推理内核并推出 MiniMax-M3 模型", section
// MSA 如何训练: top-k selection has no gradient, so a KL loss matches the Index
// Branch's distribution to the Main Branch's attention; the teacher is the Main
// Branch's distribution over the selected tokens averaged over the group's
// heads.  Per (sequence, group, query) over T (the visible tokens of the
// selected blocks and the local block):
//   teacher  p_j = (1/G) sum_h exp(scale q_h . k_j - lse_h),
//   student  s_j = softmax_j(iq . ik_j)   (raw index scores),
//   kl = sum_j p_j ln p_j - sum_j p_j z_j + ln sum_j exp(z_j),  z_j = iq . ik_j,
// with lse_h the Main Branch's log-sum-exp from the forward pass, so that the
// teacher needs no normalisation of its own and every sum splits over blocks.
//
// KV-outer over the same gather plan as the attention: persistent workgroups
// walk the tiles with K and the index keys of one block in LDS; each wave owns
// 32 rows (32 / G positions, all G heads).  S = Q K^T and Z = IQ IK^T run on
// 32x32x16 bf16 MFMA with the query rows as the M operand, so that a lane holds
// the scores of one key for 16 rows: the heads of a position sit in the lane's
// registers (and, for G >= 8, its partner lane's), and the group average is an
// in-lane sum plus one exchange.  Z is formed for every head row (the rows of a
// position read the same index-query row), which keeps it in S's layout.  Each
// (row, slot) gets a partial {sum p log2 p, sum p z, max z log2 e, sum 2^(z log2 e
// - max)}; a merge adds a row's partials.  Optionally the teacher itself is
// stored, one fp16 value per (row, slot, key of the block), for a backward
// that reads it instead of forming S again.
#include "fwd_tiles.h"

namespace msa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;

// Rows of index queries one wave keeps: 32 / G positions, at most 8 (G >= 4).
constexpr int kIqRows = 8;

// The wave's index-query rows (one per position) by direct global-to-LDS loads:
// row r at r * 2 * DIDX bytes, its 16-byte chunk c in slot c ^ (r % CPI), so the
// rows of different positions read at one chunk index fall in different bank
// groups.  `mine` points at the index-query row of this lane's position; the
// row of position u is taken from lane u * G.  Rows past the wave's positions
// fetch the last one again (allocated, never read).
template <int DIDX, int G>
__device__ __forceinline__ void fetch_iq_rows(unsigned char* iqw, const uint16_t* mine, int lane) {
  constexpr int NP = 32 / G;                       // positions per wave
  constexpr int CPI = DIDX / 8;                    // chunks per row (16 or 8)
  constexpr int RPI = 64 / CPI;                    // rows per load instruction (4 or 8)
  constexpr int NI = (NP + RPI - 1) / RPI;
  const uint64_t me = reinterpret_cast<uint64_t>(mine);
#pragma unroll
  for (int u = 0; u < NI; ++u) {
    const int r = RPI * u + lane / CPI;
    const uint64_t src = shfl_u64(me, min(r, NP - 1) * G);
    const int c = (lane % CPI) ^ (r % CPI);
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src + 16 * c),
                                     (__attribute__((address_space(3))) void*)(iqw + 1024 * u), 16, 0, 0);
  }
}

// S = Q K^T for one wave (query rows as M, keys as N): s[T] holds keys
// 32T .. 32T+31, lane column = key, register e = query row 8(e/4) + 4 half + e%4.
__device__ __forceinline__ void q_k_scores(const uint16_t* Ks, const unsigned char* qw, int lane, f32x16 (&s)[4]) {
  const int col = lane & 31, half = lane >> 5;
  const uint16_t* kbase = Ks + col * KP + 8 * half;
  const unsigned char* qbase = qw + col * 256;
  const int qsw = col & 15;
#pragma unroll
  for (int T = 0; T < 4; ++T) s[T] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const uint4 qf = *reinterpret_cast<const uint4*>(qbase + 16 * ((2 * ks + half) ^ qsw));
#pragma unroll
    for (int T = 0; T < 4; ++T)
      s[T] = mfma_32x32x16(qf, *reinterpret_cast<const uint4*>(kbase + 32 * T * KP + 16 * ks), s[T]);
  }
}

// Z = IQ IK^T in the layout of q_k_scores: the M operand row of query row r is
// the index-query row of its position r / G.
template <int DIDX, int G>
__device__ __forceinline__ void iq_ik_scores(const uint16_t* IKs, const unsigned char* iqw, int lane,
                                             f32x16 (&z)[4]) {
  constexpr int IKP = DIDX + 8;
  constexpr int CPI = DIDX / 8;
  const int col = lane & 31, half = lane >> 5;
  const int pos = col / G;
  const uint16_t* kbase = IKs + col * IKP + 8 * half;
  const unsigned char* qbase = iqw + pos * (2 * DIDX);
#pragma unroll
  for (int T = 0; T < 4; ++T) z[T] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < DIDX / 16; ++ks) {
    const uint4 qf = *reinterpret_cast<const uint4*>(qbase + 16 * ((2 * ks + half) ^ (pos % CPI)));
#pragma unroll
    for (int T = 0; T < 4; ++T)
      z[T] = mfma_32x32x16(qf, *reinterpret_cast<const uint4*>(kbase + 32 * T * IKP + 16 * ks), z[T]);
  }
}

// Lane-local positions.  A lane's 16 registers hold rows 8(e/4) + 4 half + e%4;
// the RPP consecutive registers of lane-local position j belong to one query
// position (all its heads for G = 4, half of them otherwise, the rest in the
// partner lane l ^ 32).
template <int G>
struct PosMap {
  static constexpr int RPP = G == 4 ? 4 : G / 2;   // registers per position in one lane
  static constexpr int NPL = 16 / RPP;             // positions per lane
  // wave-local position of lane-local position j
  static __device__ __forceinline__ int wpos(int j, int half) { return G == 4 ? 2 * j + half : j; }
};

struct KlAcc {
  float a, b, m, l;   // sum p log2 p, sum p z, max z log2 e, sum 2^(z log2 e - m)
};

__device__ __forceinline__ KlAcc kl_combine(KlAcc x, KlAcc y) {
  const float m = fmaxf(x.m, y.m);
  const float NEG_INF = -__builtin_huge_valf();
  const float lx = x.m == NEG_INF ? 0.f : x.l * __builtin_amdgcn_exp2f(x.m - m);
  const float ly = y.m == NEG_INF ? 0.f : y.l * __builtin_amdgcn_exp2f(y.m - m);
  return KlAcc{x.a + y.a, x.b + y.b, m, lx + ly};
}

// Visibility limit of a lane-local position for this lane's key column: key
// key0 + 32T + col is visible iff 32T <= limit.  -1 for a position without a
// row; 127 (every key) when the tile needs no mask; else the position's
// offset past the column's first key, clamped to [-1, 127].
template <bool MASKED>
__device__ __forceinline__ int key_limit(int valid, int64_t pos, int64_t key0, int col) {
  if (!valid) return -1;
  if (!MASKED) return 127;
  return (int)max<int64_t>(-1, min<int64_t>(127, pos - key0 - col));
}

// The lse (log2 units) of the 16 query rows a lane's accumulator registers
// hold (rows 8(e/4) + 4 half + e%4 of the wave's 32), through the wave's
// 32-float LDS slot: both lanes of a row (l and l ^ 32 hold the same row)
// write its value, and every lane reads its rows as four float4s (no
// shuffles).  A row that does not exist must carry +inf, so that all its
// probabilities come out exactly 0.
__device__ __forceinline__ void rows_lse(float* slot, float lse_mine, int lane, float (&lse2)[16]) {
  slot[lane & 31] = lse_mine;
  const int half = lane >> 5;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const float4 v = *reinterpret_cast<const float4*>(slot + 8 * m + 4 * half);
    lse2[4 * m] = v.x;
    lse2[4 * m + 1] = v.y;
    lse2[4 * m + 2] = v.z;
    lse2[4 * m + 3] = v.w;
  }
}

// Value x of the first head row of lane-local position j (lane wpos(j, half) * G):
// two lane reads with constant lanes, no shuffle.
template <int G>
__device__ __forceinline__ int pos_value(int x, int j, int half) {
  const int v0 = __builtin_amdgcn_readlane(x, PosMap<G>::wpos(j, 0) * G);
  const int v1 = __builtin_amdgcn_readlane(x, PosMap<G>::wpos(j, 1) * G);
  return half ? v1 : v0;
}

// Teacher probabilities of one tile for one wave: P[T][j] is the group's
// average probability of key key0 + 32T + column for lane-local position j
// (0 for keys after the position and for rows that do not exist, whose lse2
// is +inf).
template <int G, bool MASKED>
__device__ __forceinline__ void teacher_probs(const f32x16 (&s)[4], const float (&lse2)[16],
                                              const int (&lim)[PosMap<G>::NPL], float c,
                                              float (&P)[4][PosMap<G>::NPL]) {
  using PM = PosMap<G>;
#pragma unroll
  for (int T = 0; T < 4; ++T) {
#pragma unroll
    for (int j = 0; j < PM::NPL; ++j) {
      float psum = 0.f;
#pragma unroll
      for (int e = j * PM::RPP; e < (j + 1) * PM::RPP; ++e)
        psum += __builtin_amdgcn_exp2f(__builtin_fmaf(s[T][e], c, -lse2[e]));  // 0 for an absent row
      if constexpr (G >= 8) psum += wave_xor32(psum);
      const bool vis = !MASKED || 32 * T <= lim[j];
      P[T][j] = vis ? psum * (1.f / G) : 0.f;
    }
  }
}

// Fold a block's teacher probabilities and student scores into this lane's
// sums for its lane-local positions (its keys only; lanes_reduce adds the
// lanes).
template <int G, bool MASKED>
__device__ __forceinline__ void student_fold(const f32x16 (&z)[4], const float (&P)[4][PosMap<G>::NPL],
                                             const int (&lim)[PosMap<G>::NPL], KlAcc (&acc)[PosMap<G>::NPL]) {
  using PM = PosMap<G>;
  const float NEG_INF = -__builtin_huge_valf();
#pragma unroll
  for (int j = 0; j < PM::NPL; ++j) {
    KlAcc x{0.f, 0.f, NEG_INF, 0.f};
    // max of the visible scores, then the sums
#pragma unroll
    for (int T = 0; T < 4; ++T) {
      const bool vis = 32 * T <= lim[j];
      if (vis) x.m = fmaxf(x.m, z[T][j * PM::RPP] * kLog2e);
    }
#pragma unroll
    for (int T = 0; T < 4; ++T) {
      const bool vis = 32 * T <= lim[j];
      const float zz = z[T][j * PM::RPP], p = P[T][j];
      if (p > 0.f) x.a += p * __log2f(p);
      x.b += p * zz;
      if (vis) x.l += __builtin_amdgcn_exp2f(zz * kLog2e - x.m);
    }
    acc[j] = kl_combine(acc[j], x);
  }
}

// Sums over the 32 lanes of each half (the keys of a block): every lane of a
// half ends with its positions' totals.
template <int G>
__device__ __forceinline__ void lanes_reduce(KlAcc (&acc)[PosMap<G>::NPL]) {
#pragma unroll
  for (int j = 0; j < PosMap<G>::NPL; ++j) {
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) {
      KlAcc y{__shfl_xor(acc[j].a, o, 64), __shfl_xor(acc[j].b, o, 64), __shfl_xor(acc[j].m, o, 64),
              __shfl_xor(acc[j].l, o, 64)};
      acc[j] = kl_combine(acc[j], y);
    }
  }
}

// ---------------------------------------------------------------- four-wave tiles
// The same partials from four-wave workgroups on the forward's 128-row tiles
// (pt * G = 128) and its dynamic per-XCD runs: each wave's query rows stay in
// VGPRs (the next tile's loaded into the other register set while the current
// one is computed), K and the index keys of a block arrive by direct
// global-to-LDS loads, the rows are laid out so that a lane's S registers
// hold whole positions (Rows4), and Z is formed per position, not per head
// row: a 16x16x32 product whose 16 M rows repeat the wave's positions, so
// that lane (key n, k-group c) holds Z of the positions its S registers hold
// (see zpos), for the key the lane's S column is.

// K (swizzled as in stage_kv_fwd) and the index keys (row r at r * 2 DIDX
// bytes, its chunk c in slot c ^ (r % CPI)) of one block, by direct loads:
// each wave issues 8 one-KB instructions of each.  Keys at or past n_valid
// repeat key n_valid - 1.  The caller waits for vmcnt(0) and a barrier.
template <int DIDX>
__device__ __forceinline__ void stage_k_ik4(unsigned char* Ks, unsigned char* IKs, const uint16_t* k,
                                            const uint16_t* ik, int64_t k0, int64_t ik0, int n_valid) {
  constexpr int CPI = DIDX / 8;
  constexpr int KPI = 64 / CPI;  // index keys per instruction
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));  // addresses formed at each staging, not kept live along the walk
  const int wave = tid >> 6, lane = tid & 63;
  const unsigned char* kb = reinterpret_cast<const unsigned char*>(k + k0);
  const unsigned char* ib = reinterpret_cast<const unsigned char*>(ik + ik0);
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int g = 8 * wave + u;
    const int row = 4 * g + (lane >> 4);
    const int c = (lane & 15) ^ (row & 15);
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(kb + (int64_t)min(row, n_valid - 1) * 256 + 16 * c),
                                     (__attribute__((address_space(3))) void*)(Ks + 1024 * g), 16, 0, 0);
  }
  constexpr int NIK = kBk * CPI / 64 / kFWaves;  // index-key instructions per wave
#pragma unroll
  for (int u = 0; u < NIK; ++u) {
    const int g = NIK * wave + u;
    const int key = KPI * g + lane / CPI;
    const int c = (lane % CPI) ^ (key % CPI);
    __builtin_amdgcn_global_load_lds(
        reinterpret_cast<const void*>(ib + (int64_t)min(key, n_valid - 1) * (2 * DIDX) + 16 * c),
        (__attribute__((address_space(3))) void*)(IKs + 1024 * g), 16, 0, 0);
  }
}

// S = Q K^T with the query rows (registers, load_q's layout) as the A
// operand and K (swizzled LDS) as B: s[T] holds keys 32T .. 32T+31, lane
// column = key, register e = query row 8(e/4) + 4 half + e%4 of the wave.
// Same operands, order and accumulation as q_k_scores.
__device__ __forceinline__ void qk_rows(const unsigned char* Ks, const uint4 (&qf)[8], int lane, f32x16 (&s)[4]) {
  const int col = lane & 31, half = lane >> 5;
  const unsigned char* kbase = Ks + col * 256;
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
    for (int T = 0; T < 4; ++T) s[T] = mfma_32x32x16(qf[ks], kf[cb][T], s[T]);
  }
}

typedef __bf16 bf16x8k __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x4 mfma16k(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8k, a), __builtin_bit_cast(bf16x8k, b), c,
                                                 0, 0, 0);
}

// Rows of the four-wave tiles.  MFMA row m (lane column m of the query
// operand) is (position, head) = ((16/G) h + e / G, e % G) of the wave, with
// h = (m >> 2) & 1 and e = 4 (m >> 3) + (m & 3): accumulator register e of a
// lane in half h is row 8 (e / 4) + 4 h + e % 4, so for G <= 16 every head of
// a position sits in one lane's registers (the group average is an in-lane
// sum) and the two halves hold different positions.  For G = 32 the one
// position's heads are split over the halves (head 16 h + e).
template <int G>
struct Rows4 {
  static constexpr int NPL = G <= 16 ? 16 / G : 1;  // positions per lane
  static constexpr int RPP = G <= 16 ? G : 16;      // registers per position
  static __device__ __forceinline__ int pos_of(int m) {
    const int h = (m >> 2) & 1, e = 4 * (m >> 3) + (m & 3);
    return G <= 16 ? (16 / G) * h + e / G : 0;
  }
  static __device__ __forceinline__ int head_of(int m) {
    const int h = (m >> 2) & 1, e = 4 * (m >> 3) + (m & 3);
    return G <= 16 ? e % G : 16 * h + e;
  }
  // wave-local position of lane-local position j in half h
  static __device__ __forceinline__ int lpos(int j, int h) { return G <= 16 ? (16 / G) * h + j : 0; }
  // the row of head 0 of wave-local position p
  static __device__ __forceinline__ constexpr int row_of(int p) {
    if (G > 16) return 0;
    const int h = p / (16 / G), e = G * (p % (16 / G));
    return 8 * (e >> 2) + 4 * h + (e & 3);
  }
};

// Value x of head 0's row of lane-local position j (two lane reads with
// constant lanes).
template <int G>
__device__ __forceinline__ int pos_value4(int x, int j, int half) {
  const int v0 = __builtin_amdgcn_readlane(x, Rows4<G>::row_of(Rows4<G>::lpos(j, 0)));
  const int v1 = __builtin_amdgcn_readlane(x, Rows4<G>::row_of(Rows4<G>::lpos(j, 1)));
  return half ? v1 : v0;
}

// Row m of the Z product (lane (n, c) gets rows 4c + i): the wave-local
// position whose values lane-local position i of the S registers needs
// (c = 2 half + (column >= 16)); rows past a lane's positions repeat its last.
template <int G>
__device__ __forceinline__ int zpos(int m) {
  constexpr int NPL = Rows4<G>::NPL;
  return Rows4<G>::lpos(min(m & 3, NPL - 1), (m >> 3) & 1);
}

// z[T][j]: Z = IQ IK^T of lane-local position j and the lane's key 32T + col,
// from the wave's index-query rows in LDS (row p at p * 2 DIDX, chunk c in
// slot c ^ (p % CPI)) and the staged index keys.
template <int DIDX, int G>
__device__ __forceinline__ void z_scores(const unsigned char* IKs, const unsigned char* iqw, int lane,
                                         float (&z)[4][Rows4<G>::NPL]) {
  constexpr int CPI = DIDX / 8, IKS = DIDX / 32;
  const int n = lane & 15, cg = lane >> 4;
  const int pm = zpos<G>(n);
  uint4 a[IKS];
#pragma unroll
  for (int ks = 0; ks < IKS; ++ks)
    a[ks] = *reinterpret_cast<const uint4*>(iqw + pm * (2 * DIDX) + 16 * ((4 * ks + cg) ^ (pm % CPI)));
  f32x4 zt[8];
#pragma unroll
  for (int kt = 0; kt < 8; ++kt) {
    const int key = 16 * kt + n;
    zt[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < IKS; ++ks) {
      const uint4 b = *reinterpret_cast<const uint4*>(IKs + key * (2 * DIDX) + 16 * ((4 * ks + cg) ^ (key % CPI)));
      zt[kt] = mfma16k(a[ks], b, zt[kt]);
    }
  }
  const bool hi = (lane & 16) != 0;  // the lane's key 32T + col lies in key tile 2T + (col >= 16)
#pragma unroll
  for (int T = 0; T < 4; ++T) {
#pragma unroll
    for (int j = 0; j < Rows4<G>::NPL; ++j) z[T][j] = hi ? zt[2 * T + 1][j] : zt[2 * T][j];
  }
}

// Teacher weights of the tile: P[T][j] is the group's average probability of
// key key0 + 32T + col for lane-local position j (0 for keys after the
// position and for rows that do not exist, whose lse2 is +inf).
template <int G, bool MASKED>
__device__ __forceinline__ void teacher_probs4(const f32x16 (&s)[4], const float (&lse2)[16],
                                               const int (&lim)[Rows4<G>::NPL], float c,
                                               float (&P)[4][Rows4<G>::NPL]) {
  using R = Rows4<G>;
#pragma unroll
  for (int T = 0; T < 4; ++T) {
#pragma unroll
    for (int j = 0; j < R::NPL; ++j) {
      float psum = 0.f;
#pragma unroll
      for (int e = j * R::RPP; e < (j + 1) * R::RPP; ++e)
        psum += __builtin_amdgcn_exp2f(__builtin_fmaf(s[T][e], c, -lse2[e]));
      if constexpr (G > 16) psum += wave_xor32(psum);
      const bool vis = !MASKED || 32 * T <= lim[j];
      P[T][j] = vis ? psum * (1.f / G) : 0.f;
    }
  }
}

// The tile's partials for the lane's positions over the block's 128 keys (the
// 32 lanes of a half hold 4 keys each): the max of the visible student scores
// first, then the three sums with that common max, added over the half's
// lanes.  Every lane of a half ends with the totals; a position without
// visible keys gets m = -inf and l = 0.
template <int G, bool MASKED>
__device__ __forceinline__ void student_tile4(const float (&z)[4][Rows4<G>::NPL], const float (&P)[4][Rows4<G>::NPL],
                                              const int (&lim)[Rows4<G>::NPL], KlAcc (&out)[Rows4<G>::NPL]) {
  using R = Rows4<G>;
  const float NEG_INF = -__builtin_huge_valf();
#pragma unroll
  for (int j = 0; j < R::NPL; ++j) {
    auto visible = [&](int T) { return 32 * T <= lim[j]; };
    float zl[4];
#pragma unroll
    for (int T = 0; T < 4; ++T) zl[T] = z[T][j] * kLog2e;
    float m = NEG_INF;
#pragma unroll
    for (int T = 0; T < 4; ++T)
      if (visible(T)) m = fmaxf(m, zl[T]);
    m = half_max(m);
    float a = 0.f, b = 0.f, l = 0.f;
#pragma unroll
    for (int T = 0; T < 4; ++T) {
      const float p = P[T][j];
      if (p > 0.f) a += p * __log2f(p);
      b += p * z[T][j];
      if (visible(T)) l += __builtin_amdgcn_exp2f(zl[T] - m);
    }
    out[j] = KlAcc{half_sum(a), half_sum(b), m, half_sum(l)};
  }
}

template <int DIDX, int G, bool LOCAL>
__global__ __launch_bounds__(kFThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_kl_tiles4(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ iq,
    const uint16_t* __restrict__ ik, const float* __restrict__ lse, AttnWs ws, float4* __restrict__ kl_part,
    _Float16* __restrict__ teacher, Dims D) {
  using R = Rows4<G>;
  constexpr int NP = 32 / G;             // positions per wave
  constexpr int CPI = DIDX / 8;          // 16-byte chunks of an index row
  constexpr int IQB = NP * 2 * DIDX;     // bytes of one wave's index-query rows
  constexpr int NPC = NP * CPI;          // their chunks
  constexpr int NIQ = (NPC + 63) / 64;   // chunks per lane
  __shared__ __align__(16) unsigned char Ks[kBk * 256];
  __shared__ __align__(16) unsigned char IKs[kBk * 2 * DIDX];
  __shared__ __align__(16) unsigned char IQs[kFWaves][2][IQB];
  __shared__ __align__(16) float LSs[kFWaves][32];
  __shared__ int2 runs[3];
  const bool leader = threadIdx.x == 0;
  RunQueue rq;
  if (leader) {
    if constexpr (LOCAL) rq.init(ws.ctr + kXcds, D.B * D.h_kv * local_tiles<false>(D));
    else rq.init(ws.ctr, ws.tile_off[ws.n_bins]);
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
  const int ps = wave * NP + R::pos_of(col), hh = R::head_of(col);  // this lane's query row
  const float c = D.scale_log2;
  auto q_ptr = [&](const TileRow& tr) {  // rows that do not exist read row 0 of the group
    const int b = tr.bg / D.h_kv, g = tr.bg % D.h_kv, i = tr.valid ? tr.i : 0;
    return q + (((int64_t)b * D.n_q + i) * D.h_q + g * G + hh) * kHeadDim;
  };
  auto lse_of = [&](const TileRow& tr) {
    const int b = tr.bg / D.h_kv, g = tr.bg % D.h_kv, i = tr.valid ? tr.i : 0;
    return lse[((int64_t)b * D.h_q + g * G + hh) * D.n_q + i];
  };
  // this lane's chunks of the wave's index-query rows of tile tr (position p's
  // row from the lane of its head 0; rows that do not exist read row 0)
  auto load_iq = [&](const TileRow& tr, uint4 (&x)[NIQ]) {
    const int b = tr.bg / D.h_kv, g = tr.bg % D.h_kv;
    const int i_mine = tr.valid ? tr.i : 0;
#pragma unroll
    for (int u = 0; u < NIQ; ++u) {
      const int pc = min(lane + 64 * u, NPC - 1);
      const int p = pc / CPI, ch = pc % CPI;
      const int i = __shfl(i_mine, R::row_of(p), 64);
      x[u] = *reinterpret_cast<const uint4*>(iq + (((int64_t)b * D.n_q + i) * D.h_kv + g) * DIDX + 8 * ch);
    }
  };
  auto store_iq = [&](unsigned char* dst, const uint4 (&x)[NIQ]) {
#pragma unroll
    for (int u = 0; u < NIQ; ++u) {
      const int pc = lane + 64 * u;
      const int p = pc / CPI, ch = pc % CPI;
      if (pc < NPC) *reinterpret_cast<uint4*>(dst + p * (2 * DIDX) + 16 * (ch ^ (p % CPI))) = x[u];
    }
  };
  auto after = [&](int t, int t1) {  // as in k_attn_tiles
    if (t1 < 0) return -1;
    if (t + 1 < run.y) return t1 + 1 < run.y ? t1 + 1 : nrun.x;
    return t1 + 1 < nrun.y ? t1 + 1 : -2;
  };

  int t = run.x;
  TileRow cur = tile_row<LOCAL, false>(tile_raw<LOCAL>(ws, D, t, ps), D, ws, t, ps);
  int t1 = t + 1 < run.y ? t + 1 : nrun.x;
  TileRaw raw1 = t1 >= 0 ? tile_raw<LOCAL>(ws, D, t1, ps) : TileRaw{-1, 0};
  uint4 qa[8], qb[8];
  load_q(q_ptr(cur), half, qa);
  float lse_cur = lse_of(cur);
  {
    uint4 x[NIQ];
    load_iq(cur, x);
    store_iq(IQs[wave][0], x);
  }
  int buf = 0;
  int staged_bg = -1, staged_t = -1;
  bool fresh = true;

  auto step = [&](uint4 (&qc)[8], uint4 (&qn)[8]) -> bool {
    if (cur.bg != staged_bg || cur.t != staged_t) {  // uniform
      if (!fresh) lds_barrier();                    // every wave is done with the staged block
      const int b = cur.bg / D.h_kv, g = cur.bg % D.h_kv;
      const int64_t k0 = (((int64_t)b * D.h_kv + g) * D.n_kv + (int64_t)cur.t * kBk) * kHeadDim;
      const int64_t ik0 = ((int64_t)b * D.n_kv + (int64_t)cur.t * kBk) * DIDX;
      stage_k_ik4<DIDX>(Ks, IKs, k, ik, k0, ik0, LOCAL ? max(1, min(kBk, D.n_kv - cur.t * kBk)) : kBk);
      __builtin_amdgcn_s_waitcnt(kWaitVm0);  // this wave's direct loads have landed
      lds_barrier();
      staged_bg = cur.bg;
      staged_t = cur.t;
    }
    fresh = false;
    const bool last = t + 1 >= run.y;  // t ends its run (uniform)
    if (leader && last && t1 >= 0) runs[(ri + 2) % 3] = rq.resolve();
    // Z before S where that keeps the registers within two waves per SIMD
    // (its 8 accumulator tiles are folded to the lane's values before S's are
    // live); for d_idx 128 and G <= 8 after S and the next tile's loads,
    // where that order does
    constexpr bool kZFirst = !(DIDX == 128 && G <= 8);
    float z[4][R::NPL];
    if constexpr (kZFirst) z_scores<DIDX, G>(IKs, IQs[wave][buf], lane, z);
    f32x16 s[4];
    qk_rows(Ks, qc, lane, s);
    const bool more = t1 >= 0;  // uniform
    TileRow nxt = cur;
    if (more) nxt = tile_row<LOCAL, false>(raw1, D, ws, t1, ps);
    uint4 xiq[NIQ];
    float lse_nxt = 0.f;
    if (more) {
      load_q(q_ptr(nxt), half, qn);
      load_iq(nxt, xiq);
      lse_nxt = lse_of(nxt);
    }
    int t2 = after(t, t1);
    TileRaw raw2{-1, 0};
    if (t2 >= 0) raw2 = tile_raw<LOCAL>(ws, D, t2, ps);
    if constexpr (!kZFirst) z_scores<DIDX, G>(IKs, IQs[wave][buf], lane, z);

    float lse2[16];  // the lse of the 16 rows this lane's registers hold (+inf: no such row)
    rows_lse(LSs[wave], cur.valid ? lse_cur * kLog2e : __builtin_huge_valf(), lane, lse2);
    int lim[R::NPL], pi[R::NPL], pv[R::NPL], pslot[R::NPL];
#pragma unroll
    for (int j = 0; j < R::NPL; ++j) {
      pi[j] = pos_value4<G>(cur.i, j, half);
      pv[j] = pos_value4<G>((int)cur.valid, j, half);
      pslot[j] = pos_value4<G>(cur.s, j, half);
      lim[j] = key_limit<LOCAL>(pv[j], D.offset + pi[j], (int64_t)cur.t * kBk, col);
    }
    float P[4][R::NPL];
    teacher_probs4<G, LOCAL>(s, lse2, lim, c, P);
    if (teacher) {  // uniform; for G = 32 both halves hold the same weights and split the key ranges
#pragma unroll
      for (int j = 0; j < R::NPL; ++j) {
        if (!pv[j]) continue;
        _Float16* dst = teacher + (((int64_t)cur.bg * D.n_q + pi[j]) * (D.k + 1) + pslot[j]) * kBk + col;
#pragma unroll
        for (int T = 0; T < 4; ++T)
          if (G <= 16 || (T >> 1) == half) dst[32 * T] = (_Float16)P[T][j];
      }
    }
    KlAcc acc[R::NPL];
    student_tile4<G, LOCAL>(z, P, lim, acc);
#pragma unroll
    for (int j = 0; j < R::NPL; ++j) {
      const bool writer = col == 0 && (G <= 16 || half == 0);  // every lane of a half holds the totals
      if (writer && pv[j]) {
        const int64_t row = (int64_t)cur.bg * D.n_q + pi[j];
        kl_part[row * (D.k + 1) + pslot[j]] = make_float4(acc[j].a, acc[j].b, acc[j].m, acc[j].l);
      }
    }
    if (!more) return false;
    // the next tile's index-query rows into the other buffer (this wave's own
    // region: its reads of this tile's rows, above, come first in LDS order)
    buf ^= 1;
    store_iq(IQs[wave][buf], xiq);
    if (last) {  // t1 starts the next run
      lds_barrier();
      fresh = true;
      run = nrun;
      nrun = uniform2(runs[(ri + 2) % 3]);
      ++ri;
      if (leader && nrun.x >= 0) rq.prefetch();
      if (t2 == -2) {  // the next run holds one tile: the one after it starts the run now known
        t2 = nrun.x;
        if (t2 >= 0) raw2 = tile_raw<LOCAL>(ws, D, t2, ps);
      }
    }
    t = t1;
    t1 = t2;
    raw1 = raw2;
    cur = nxt;
    lse_cur = lse_nxt;
    return true;
  };
  while (step(qa, qb) && step(qb, qa)) {
  }
}

// 32 lanes per (sequence, group, query): lane j takes slots j, j + 32, .. of
// the row's partials (the listed non-local blocks, and the local block, slot
// k; the other slots add nothing), adds its own in slot order, and the 32
// lanes' sums are added in a fixed tree order (the max first, then the
// rescaled sums); lane 0 forms the KL value.
__global__ __launch_bounds__(256) void k_kl_merge(const int32_t* __restrict__ block_idx,
                                                  const float4* __restrict__ kl_part, float* __restrict__ kl,
                                                  float* __restrict__ lse_index, Dims D) {
  const int64_t row = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 5;
  const int j = threadIdx.x & 31;
  const int64_t rows = (int64_t)D.B * D.h_kv * D.n_q;
  const bool live = row < rows;  // whole half-waves: a row's 32 lanes agree
  const float NEG_INF = -__builtin_huge_valf();
  KlAcc acc{0.f, 0.f, NEG_INF, 0.f};
  if (live) {
    const int i = (int)(row % D.n_q);
    const int local = (int)((D.offset + i) / kBk);
    const int32_t* sel = block_idx + row * D.k;
    const float4* part = kl_part + row * (D.k + 1);
    for (int s = j; s <= D.k; s += 32) {
      if (s == D.k || nonlocal_slot(sel, s, local)) {
        const float4 x = part[s];
        acc = kl_combine(acc, KlAcc{x.x, x.y, x.z, x.w});
      }
    }
  }
  // the lanes' maximum, then every lane's sums at that maximum, added over the 32 lanes
  float m = acc.m;
#pragma unroll
  for (int o = 1; o < 32; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  float l = acc.m == NEG_INF ? 0.f : acc.l * __builtin_amdgcn_exp2f(acc.m - m);
  float a = acc.a, b = acc.b;
#pragma unroll
  for (int o = 1; o < 32; o <<= 1) {
    a += __shfl_xor(a, o, 64);
    b += __shfl_xor(b, o, 64);
    l += __shfl_xor(l, o, 64);
  }
  if (live && j == 0) {
    const float lz = (m + __log2f(l)) * kLn2;  // the student's log-normaliser
    kl[row] = a * kLn2 - b + lz;
    if (lse_index) lse_index[row] = lz;
  }
}

// ---------------------------------------------------------------- dense mode
// The KL value over every visible token (the indexer warmup, where both
// branches run full attention: page "MiniMax 发布 MSA…", section MSA 如何训练),
// with lse from the dense attention.  Query-outer like the dense attention:
// a workgroup owns pt aligned positions of one (sequence, group) and streams
// blocks 0 .. its own; K and the index keys of block t+1 are loaded into
// registers while block t is computed.  Each lane sums over its keys across
// all blocks; one reduction over the lanes at the end gives the row's value,
// so there are no partials.
template <int DIDX>
struct KIkRegs {  // native vectors: whole-register copies, so the struct stays in registers
  u32x4 kr[2048 / kThreads];
  u32x4 ir[kBk * (DIDX / 8) / kThreads];
};

template <int DIDX>
__device__ __forceinline__ void k_ik_load(KIkRegs<DIDX>& x, const uint16_t* __restrict__ kb,
                                          const uint16_t* __restrict__ ikb, int n_valid) {
  constexpr int CPI = DIDX / 8;
  constexpr int KPER = 2048 / kThreads, IPER = kBk * CPI / kThreads;
  const int tid = threadIdx.x;
  const char* kbase = reinterpret_cast<const char*>(kb);
  const char* ibase = reinterpret_cast<const char*>(ikb);
#pragma unroll
  for (int u = 0; u < KPER; ++u) {
    const int c = tid + kThreads * u;
    x.kr[u] = *reinterpret_cast<const u32x4*>(kbase + (uint32_t)min(c >> 4, n_valid - 1) * 256u + 16u * (c & 15));
  }
#pragma unroll
  for (int u = 0; u < IPER; ++u) {
    const int c = tid + kThreads * u;
    x.ir[u] = *reinterpret_cast<const u32x4*>(ibase + (uint32_t)min(c / CPI, n_valid - 1) * (2u * DIDX) +
                                              16u * (c % CPI));
  }
}

template <int DIDX>
__device__ __forceinline__ void k_ik_store(uint16_t* Ks, uint16_t* IKs, const KIkRegs<DIDX>& x) {
  constexpr int IKP = DIDX + 8;
  constexpr int CPI = DIDX / 8;
  constexpr int KPER = 2048 / kThreads, IPER = kBk * CPI / kThreads;
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < KPER; ++u) {
    const int c = tid + kThreads * u;
    *reinterpret_cast<u32x4*>(Ks + (c >> 4) * KP + (c & 15) * 8) = x.kr[u];
  }
#pragma unroll
  for (int u = 0; u < IPER; ++u) {
    const int c = tid + kThreads * u;
    *reinterpret_cast<u32x4*>(IKs + (c / CPI) * IKP + (c % CPI) * 8) = x.ir[u];
  }
}

template <int DIDX, int G>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_kl_dense(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ iq,
    const uint16_t* __restrict__ ik, const float* __restrict__ lse, float* __restrict__ kl,
    float* __restrict__ lse_index, Dims D) {
  using PM = PosMap<G>;
  constexpr int IKP = DIDX + 8;
  __shared__ __align__(16) uint16_t Ks[kBk * KP];
  __shared__ __align__(16) uint16_t IKs[kBk * IKP];
  __shared__ __align__(16) unsigned char Qs[kWaves][kQRegion];
  __shared__ __align__(16) unsigned char IQs[kWaves][kIqRows * 2 * DIDX];
  __shared__ __align__(16) float LSs[kWaves][32];

  const int nbg = D.B * D.h_kv;
  const int n_t = (int)((D.offset + D.n_q - 1) / D.pt - D.offset / D.pt + 1);
  const int bg = blockIdx.x % nbg;
  const int tile = n_t - 1 - (int)(blockIdx.x / nbg);   // heaviest first
  const int b = bg / D.h_kv, g = bg % D.h_kv;
  const int p0 = (int)((D.offset / D.pt + tile) * D.pt);
  const int t_last = p0 / kBk;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 31, half = lane >> 5;
  const int r = wave * 32 + col;
  const int ps = r / G, hh = r % G;
  const int pos = p0 + ps;
  const bool valid = ps < D.pt && pos >= D.offset && pos < D.offset + D.n_q;
  const int i = valid ? (int)(pos - D.offset) : 0;
  unsigned char* qw = Qs[wave];
  unsigned char* iqw = IQs[wave];
  const float c = D.scale_log2;

  fetch_q_rows(qw, q + (((int64_t)b * D.n_q + i) * D.h_q + g * G + hh) * kHeadDim, lane);
  fetch_iq_rows<DIDX, G>(iqw, iq + (((int64_t)b * D.n_q + i) * D.h_kv + g) * DIDX, lane);
  const float lse_mine = lse[((int64_t)b * D.h_q + g * G + hh) * D.n_q + i] * kLog2e;
  float lse2[16];
  rows_lse(LSs[wave], valid ? lse_mine : __builtin_huge_valf(), lane, lse2);
  int64_t ppos[PM::NPL];  // position of each lane-local position
  int pi[PM::NPL], pv[PM::NPL];
#pragma unroll
  for (int j = 0; j < PM::NPL; ++j) {
    pi[j] = pos_value<G>(i, j, half);
    pv[j] = pos_value<G>((int)valid, j, half);
    ppos[j] = D.offset + pi[j];
  }

  const uint16_t* kg = k + ((int64_t)b * D.h_kv + g) * D.n_kv * kHeadDim;
  const uint16_t* ikg = ik + (int64_t)b * D.n_kv * DIDX;
  auto n_valid = [&](int t) { return max(1, min(kBk, D.n_kv - t * kBk)); };
  {
    KIkRegs<DIDX> x;
    k_ik_load<DIDX>(x, kg, ikg, n_valid(0));
    k_ik_store<DIDX>(Ks, IKs, x);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);  // this wave's query and index-query rows have landed
    __syncthreads();
  }
  KlAcc acc[PM::NPL];
#pragma unroll
  for (int j = 0; j < PM::NPL; ++j) acc[j] = KlAcc{0.f, 0.f, -__builtin_huge_valf(), 0.f};
  for (int t = 0; t <= t_last; ++t) {
    const bool more = t < t_last;
    KIkRegs<DIDX> x;
    if (more)
      k_ik_load<DIDX>(x, kg + (int64_t)(t + 1) * kBk * kHeadDim, ikg + (int64_t)(t + 1) * kBk * DIDX, n_valid(t + 1));
    const int64_t key0 = (int64_t)t * kBk;
    int lim[PM::NPL];
#pragma unroll
    for (int j = 0; j < PM::NPL; ++j) lim[j] = key_limit<true>(pv[j], ppos[j], key0, col);
    float P[4][PM::NPL];
    {
      f32x16 sc[4];
      q_k_scores(Ks, qw, lane, sc);
      if (t == t_last) teacher_probs<G, true>(sc, lse2, lim, c, P);
      else teacher_probs<G, false>(sc, lse2, lim, c, P);
    }
    {
      f32x16 zz[4];
      iq_ik_scores<DIDX, G>(IKs, iqw, lane, zz);
      if (t == t_last) student_fold<G, true>(zz, P, lim, acc);
      else student_fold<G, false>(zz, P, lim, acc);
    }
    __syncthreads();  // every wave is done with block t
    if (more) {
      k_ik_store<DIDX>(Ks, IKs, x);
      __syncthreads();
    }
  }
  lanes_reduce<G>(acc);
#pragma unroll
  for (int j = 0; j < PM::NPL; ++j) {
    const bool writer = col == PM::wpos(j, half) * G && (G == 4 || half == 0);
    if (writer && pv[j]) {
      const float lz = (acc[j].m + __log2f(acc[j].l)) * kLn2;
      kl[(int64_t)bg * D.n_q + pi[j]] = acc[j].a * kLn2 - acc[j].b + lz;
      if (lse_index) lse_index[(int64_t)bg * D.n_q + pi[j]] = lz;
    }
  }
}

}  // namespace

bool kl_supported(const Dims& D) {
  return (D.G == 4 || D.G == 8 || D.G == 16 || D.G == 32) && D.idx_eb == 2 && D.kv_eb == 2 && !dims_varlen(D);
}

hipError_t launch_index_kl(const uint16_t* q, const uint16_t* k, const uint16_t* index_q, const uint16_t* index_k,
                           const int32_t* block_idx, const float* lse, float* kl, float* lse_index, uint16_t* teacher,
                           const AttnWs& ws, float4* kl_part, const Dims& D, hipStream_t stream) {
  const Dims F = fwd_attn_dims(D);  // 128-row tiles
  hipError_t e = launch_gather_plan(block_idx, ws, F, stream);
  if (e != hipSuccess) return e;
  const dim3 grid(2 * persistent_grid()), block(kFThreads);  // two four-wave workgroups per CU
  auto go = [&](auto didx, auto g) {
    constexpr int DI = decltype(didx)::value, GG = decltype(g)::value;
    _Float16* t = reinterpret_cast<_Float16*>(teacher);
    hipLaunchKernelGGL((k_kl_tiles4<DI, GG, false>), grid, block, 0, stream, q, k, index_q, index_k, lse, ws,
                       kl_part, t, F);
    hipLaunchKernelGGL((k_kl_tiles4<DI, GG, true>), grid, block, 0, stream, q, k, index_q, index_k, lse, ws,
                       kl_part, t, F);
  };
  using I128 = std::integral_constant<int, 128>;
  using I64 = std::integral_constant<int, 64>;
  auto by_g = [&](auto didx) {
    switch (D.G) {
      case 4: go(didx, std::integral_constant<int, 4>{}); break;
      case 8: go(didx, std::integral_constant<int, 8>{}); break;
      case 16: go(didx, std::integral_constant<int, 16>{}); break;
      default: go(didx, std::integral_constant<int, 32>{}); break;
    }
  };
  if (D.d_idx == 128) by_g(I128{}); else by_g(I64{});
  const int64_t rows = (int64_t)D.B * D.h_kv * D.n_q;
  hipLaunchKernelGGL(k_kl_merge, dim3((unsigned)((rows * 32 + 255) / 256)), dim3(256), 0, stream, block_idx, kl_part,
                     kl, lse_index, D);
  return hipGetLastError();
}

hipError_t launch_dense_index_kl(const uint16_t* q, const uint16_t* k, const uint16_t* index_q,
                                 const uint16_t* index_k, const float* lse, float* kl, float* lse_index,
                                 const Dims& D, hipStream_t stream) {
  const int64_t n_t = (D.offset + D.n_q - 1) / D.pt - D.offset / D.pt + 1;
  const dim3 grid((unsigned)((int64_t)D.B * D.h_kv * n_t)), block(kThreads);
  auto go = [&](auto didx, auto g) {
    constexpr int DI = decltype(didx)::value, GG = decltype(g)::value;
    hipLaunchKernelGGL((k_kl_dense<DI, GG>), grid, block, 0, stream, q, k, index_q, index_k, lse, kl, lse_index, D);
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
  return hipGetLastError();
}

}  // namespace msa
