// Shared device helpers and launch descriptors of the MSA kernels (gfx950).
#pragma once
#include <type_traits>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

constexpr int kBk = 128;        // block size the kernels are built for
constexpr int kHeadDim = 128;   // main-branch head dim
constexpr int kMaxTopk = 64;    // one selection per wavefront lane at most
constexpr int kTileRows = 256;  // query rows (positions x heads) per attention tile (8 waves x 32)
constexpr int kMaxGroup = 128;  // query heads per KV head
constexpr int kChunkRows = 1024;   // query rows per gather-plan workgroup
constexpr int kGroupChunks = 8;    // plan chunks per gather-list group (8192 query rows)
constexpr int kMaxPlanBlocks = 16384;  // LDS histogram bins of the gather plan (n_kv <= 2M)
constexpr int kPoolStage = 8;          // pooled scores a lane stages before one 32-byte store
constexpr int kRowsMaxQ = 4;           // query rows per sequence up to which attention runs query-outer
constexpr int kRowsPart = 16 * kHeadDim + 16;  // floats per query-outer partial: o[16][d], lse[16]
constexpr int kWorkCounters = 16;      // per-XCD run counters: 8 for the tiles, 8 for the local/merge pass

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Eight FP8 E4M3 codes (bytes 0..7 of w) widened to eight bf16, in order.
// Every E4M3 value is a bf16 value, so the conversion (scale 1) is exact.
__device__ __forceinline__ u32x4 e4m3x8_to_bf16(uint2 w) {
  return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.0f, true)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.0f, true))};
}

// s_waitcnt immediates (gfx9 encoding: vmcnt [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8])
constexpr int kWaitVm0 = 0x0F70;    // vmcnt(0)
constexpr int kWaitLgkm0 = 0xC07F;  // lgkmcnt(0)

// Word 3 of a gfx9 raw buffer descriptor (stride 0, byte-addressed records):
// a 32-bit data format, so the range check is on bytes, offset < record count.
constexpr int kRawBufferFlags = 0x00020000;

// Problem dimensions as the kernels see them (all derived on the host).
struct Dims {
  int32_t B, n_q, n_kv, h_q, h_kv, G, d, d_idx, k, n_blk;
  int32_t pt;          // query positions per attention tile (power of two, pt * G <= 256, pt <= 128)
  int64_t offset;      // position of query row 0 (uniform batches)
  float scale;         // softmax scale
  float scale_log2;    // softmax scale * log2(e)
  int32_t idx_eb;      // bytes per index_q / index_k element: 2 (bf16) or 1 (FP8 E4M3)
  int32_t kv_eb;       // bytes per k / v element: 2 (bf16) or 1 (FP8 E4M3)
  // Variable-length batches and paged caches.  All null: every sequence has
  // n_q query rows at positions offset .. offset + n_q - 1 and n_kv cached
  // tokens, each tensor contiguous.  Otherwise n_q and n_kv are maxima, per-row
  // outputs keep n_q rows per (sequence, group) of which the first qo_len are
  // written, and a sequence's queries sit at the end of its cache.
  const int32_t* qo_lens;   // [B] query rows per sequence (null: n_q each)
  const int32_t* kv_lens;   // [B] cached tokens per sequence (null: n_kv each)
  const int32_t* q_starts;  // [B] first row of each sequence in the packed q, index_q, out (null: b * n_q)
  const int32_t* pages;     // [B][pages_per_seq] physical page (= block) of each logical block (null: contiguous)
  int32_t pages_per_seq;
  int32_t num_pages;        // pages in the k, v and index_k pools
  int32_t total_q;          // rows of the packed q, index_q and out
};

// Per-sequence view.  Lengths are clamped to the maxima the launch was sized
// for and an out-of-range page to the pool, so malformed length or page data
// gives wrong results for that sequence but never an access outside the
// buffers.
__device__ __forceinline__ int seq_nkv(const Dims& D, int b) {
  return D.kv_lens ? max(0, min(D.kv_lens[b], D.n_kv)) : D.n_kv;
}
__device__ __forceinline__ int seq_nq(const Dims& D, int b) {
  return D.qo_lens ? max(0, min(min(D.qo_lens[b], D.n_q), seq_nkv(D, b))) : D.n_q;
}
// position of the sequence's query row 0
__device__ __forceinline__ int64_t seq_offset(const Dims& D, int b) {
  return D.qo_lens || D.kv_lens ? (int64_t)seq_nkv(D, b) - seq_nq(D, b) : D.offset;
}
// row of query i of sequence b in the packed q / index_q / out
__device__ __forceinline__ int64_t q_row(const Dims& D, int b, int i) {
  if (!D.q_starts) return (int64_t)b * D.n_q + i;
  return min((int64_t)max(D.q_starts[b], 0) + i, (int64_t)D.total_q - 1);
}
// physical page of logical block t of sequence b
__device__ __forceinline__ int64_t kv_page(const Dims& D, int b, int t) {
  const int tt = min(max(t, 0), D.pages_per_seq - 1);
  return min(max(D.pages[(int64_t)b * D.pages_per_seq + tt], 0), D.num_pages - 1);
}
// element offset of the first key of block t, KV head g, in k / v
__device__ __forceinline__ int64_t kv_block_off(const Dims& D, int b, int g, int t) {
  if (D.pages) return (kv_page(D, b, t) * D.h_kv + g) * (int64_t)kBk * kHeadDim;
  return (((int64_t)b * D.h_kv + g) * D.n_kv + (int64_t)t * kBk) * kHeadDim;
}
// element offset of the first key of block t in index_k
__device__ __forceinline__ int64_t ik_block_off(const Dims& D, int b, int t) {
  if (D.pages) return kv_page(D, b, t) * (int64_t)kBk * D.d_idx;
  return ((int64_t)b * D.n_kv + (int64_t)t * kBk) * D.d_idx;
}

// The same views for kernels instantiated twice: VL = false is the uniform,
// contiguous case with no per-sequence lookups at all.
inline bool dims_varlen(const Dims& D) { return D.qo_lens || D.kv_lens || D.q_starts || D.pages; }
template <bool VL> __device__ __forceinline__ int nq_of(const Dims& D, int b) {
  if constexpr (VL) return seq_nq(D, b); else return D.n_q;
}
template <bool VL> __device__ __forceinline__ int nkv_of(const Dims& D, int b) {
  if constexpr (VL) return seq_nkv(D, b); else return D.n_kv;
}
template <bool VL> __device__ __forceinline__ int64_t off_of(const Dims& D, int b) {
  if constexpr (VL) return seq_offset(D, b); else return D.offset;
}
template <bool VL> __device__ __forceinline__ int64_t qrow_of(const Dims& D, int b, int i) {
  if constexpr (VL) return q_row(D, b, i); else return (int64_t)b * D.n_q + i;
}
template <bool VL> __device__ __forceinline__ int64_t kvoff_of(const Dims& D, int b, int g, int t) {
  if constexpr (VL) return kv_block_off(D, b, g, t);
  else return (((int64_t)b * D.h_kv + g) * D.n_kv + (int64_t)t * kBk) * kHeadDim;
}
template <bool VL> __device__ __forceinline__ int64_t ikoff_of(const Dims& D, int b, int t) {
  if constexpr (VL) return ik_block_off(D, b, t); else return ((int64_t)b * D.n_kv + (int64_t)t * kBk) * D.d_idx;
}

// Workspace carve-up of the sparse attention stage (device pointers).
struct AttnWs {
  int32_t* hist;       // [B*h_kv][n_ch][n_blk] per-chunk block histograms, then chunk offsets
  int32_t* cnt;        // [bins]   gathered rows per bin (b, g, query group, block)
  int32_t* bsum;       // [2 * scan blocks] block sums of the two-level scan
  int32_t* off;        // [bins+1] exclusive scan of cnt
  int32_t* tile_off;   // [bins+1] exclusive scan of ceil(cnt / pt); last = tile count
  int2* list;          // [max_tiles * pt] {row-slot id i * k + s (-1 = empty), bin of the tile}, tile-major
  float* part_lse;     // [B*h_kv*n_q*(k+1)][G]     base-2 log-sum-exp of each non-local partial (-inf: none)
  uint32_t* part_o;    // [B*h_kv*n_q*(k+1)][12][G][4] normalised partials, 12-bit block-scaled codes, chunk-major
  uint16_t* part_ex;   // [B*h_kv*n_q*(k+1)][G][2]     their exponents, one byte per 32-value group
  int32_t* ctr;        // [kWorkCounters] work counters of the forward attention kernels (zeroed by the plan)
  int64_t max_tiles;
  int64_t n_bins;      // B * h_kv * query groups * n_blk
  int32_t n_groups;    // query groups per (b, g)
};

// Is slot s of a block_idx row a non-local block with a partial of its own?
// Rows are ascending; a repeated entry is ignored; the local block and
// anything past it carry no partial.
__device__ __forceinline__ bool nonlocal_slot(const int32_t* row, int s, int local) {
  const int t = row[s];
  return t >= 0 && t < local && (s == 0 || row[s - 1] != t);
}

// 32x32x16 bf16 MFMA, fp32 accumulate.  Operands are 8 packed bf16 per lane.
__device__ __forceinline__ f32x16 mfma_32x32x16(uint4 a, uint4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// FP8 (OCP E4M3) operands: 32 packed values per lane.  The gfx950 f8f6f4 MFMAs
// with format code 0 for both operands and no block scale: products of E4M3
// values are exact in fp32, accumulation is fp32.  Lane l supplies row (or
// column) l % M and bytes [32 * (l / M), 32 * (l / M) + 32) of the k-step, with
// the same k-order in A and B; the accumulator layout is that of the bf16 MFMA
// of the same M.
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x16 mfma_f8_32x32x64(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f8_16x16x128(i32x8 a, i32x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
// Two 16-byte pieces as one 32-byte operand.
__device__ __forceinline__ i32x8 join32(u32x4 lo, u32x4 hi) {
  return __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// x of lane l ^ 32 (v_permlane32_swap: the upper 32 lanes of one copy of x
// trade places with the lower 32 of another; no LDS round trip).
__device__ __forceinline__ float wave_xor32(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);  // {x of lanes 0-31, x of lanes 32-63}
  return __builtin_bit_cast(float, (threadIdx.x & 32) ? r[0] : r[1]);
}

// Reduction over the 32 lanes of each half-wave with DPP moves inside rows of
// 16 lanes (xor 1 and xor 2 by quad permutes, then the half-row and row
// mirrors), after which every lane of a row holds its row's total, and one
// row swap that combines the two rows of each half.  No LDS round trip; every
// lane of a half gets the same value (op is commutative and exact in either
// order).
// Needs all 64 lanes active.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
// Reduction over each row of 16 lanes (DPP only): every lane of a row gets
// the same value, since each step combines a lane with its partner in both
// orders of a commutative op.
template <typename Op>
__device__ __forceinline__ float row16_reduce(float x, Op op) {
  x = op(x, dpp_move<0xB1>(x));   // quad_perm [1, 0, 3, 2]
  x = op(x, dpp_move<0x4E>(x));   // quad_perm [2, 3, 0, 1]
  x = op(x, dpp_move<0x141>(x));  // row_half_mirror
  return op(x, dpp_move<0x140>(x));  // row_mirror
}
template <typename Op>
__device__ __forceinline__ float half_reduce(float x, Op op) {
  x = op(x, dpp_move<0xB1>(x));   // quad_perm [1, 0, 3, 2]
  x = op(x, dpp_move<0x4E>(x));   // quad_perm [2, 3, 0, 1]
  x = op(x, dpp_move<0x141>(x));  // row_half_mirror
  x = op(x, dpp_move<0x140>(x));  // row_mirror
  // the other row of the half: v_permlane16_swap trades the odd rows of one
  // copy of x with the even rows of another ({rows 0, 0, 2, 2} and {rows 1,
  // 1, 3, 3}); each lane takes the one that is not its own row (a select: the
  // compiler is known to mistake the two results for one when both feed one op)
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return op(x, __builtin_bit_cast(float, (threadIdx.x & 16) ? r[0] : r[1]));
}
__device__ __forceinline__ float half_max(float x) {
  return half_reduce(x, [](float a, float b) { return fmaxf(a, b); });
}
__device__ __forceinline__ float half_sum(float x) {
  return half_reduce(x, [](float a, float b) { return a + b; });
}

// A 32x32 MFMA accumulator register e of lane l holds row 8*(e/4) + 4*(l/32) + e%4,
// column l%32.
__device__ __forceinline__ int acc_row(int e, int lane) { return 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3); }

}  // namespace msa
