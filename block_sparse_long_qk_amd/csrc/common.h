// Shared device helpers and launch descriptors of the MSA kernels (gfx950).
#pragma once
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

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// s_waitcnt immediates (gfx9 encoding: vmcnt [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8])
constexpr int kWaitVm0 = 0x0F70;    // vmcnt(0)
constexpr int kWaitLgkm0 = 0xC07F;  // lgkmcnt(0)

// Problem dimensions as the kernels see them (all derived on the host).
struct Dims {
  int32_t B, n_q, n_kv, h_q, h_kv, G, d, d_idx, k, n_blk;
  int32_t pt;          // query positions per attention tile (power of two, pt * G <= 256, pt <= 128)
  int64_t offset;      // position of query row 0
  float scale;         // softmax scale
  float scale_log2;    // softmax scale * log2(e)
};

// Workspace carve-up of the sparse attention stage (device pointers).
struct AttnWs {
  int32_t* hist;       // [B*h_kv][n_ch][n_blk] per-chunk block histograms, then chunk offsets
  int32_t* cnt;        // [bins]   gathered rows per bin (b, g, query group, block)
  int32_t* bsum;       // [2 * scan blocks] block sums of the two-level scan
  int32_t* off;        // [bins+1] exclusive scan of cnt
  int32_t* tile_off;   // [bins+1] exclusive scan of ceil(cnt / pt); last = tile count
  int2* list;          // [max_tiles * pt] {row-slot id i * k + s (-1 = empty), bin of the tile}, tile-major
  float* part_lse;     // [B*h_kv*n_q*(k+1)][G]     base-2 log-sum-exp of each non-local partial (-inf: none)
  uint16_t* part_o;    // [B*h_kv*n_q*(k+1)][16][G][8] normalised partials, bf16, chunk-major per block
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

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ float wave_xor32(float x) { return __shfl_xor(x, 32, 64); }

// A 32x32 MFMA accumulator register e of lane l holds row 8*(e/4) + 4*(l/32) + e%4,
// column l%32.
__device__ __forceinline__ int acc_row(int e, int lane) { return 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3); }

}  // namespace msa
