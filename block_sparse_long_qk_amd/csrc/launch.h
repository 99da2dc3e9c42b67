// Kernel launchers of the MSA forward pass (host side, internal).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace msa {

// Timing marks (msa_forward_marked): records an event on `stream` after a
// kernel launch, named `name`, when the calling thread is inside a marked
// call; otherwise does nothing.
void mark(const char* name, hipStream_t stream);

// Index scores + block max-pool: pooled[B][h_kv][n_q][n_blk] (fp32).
// index_q / index_k elements are bf16 or E4M3 bytes (Dims::idx_eb).
hipError_t launch_index_scores(const void* index_q, const void* index_k, float* pooled, const Dims& D,
                               hipStream_t stream);

// Index scores with the block top-k fused into the epilogue (no pooled
// round-trip); possible when one launch covers every block of every row.
bool index_topk_fusable(const Dims& D);
hipError_t launch_index_topk(const void* index_q, const void* index_k, int32_t* block_idx, const Dims& D,
                             hipStream_t stream);

// Exp-free block top-k with the forced local block: block_idx[B][h_kv][n_q][k].
hipError_t launch_block_topk(const float* pooled, int32_t* block_idx, const Dims& D, hipStream_t stream);

// Gather plan: per (b, g, block) lists of row-slot ids and the tile list.
hipError_t launch_gather_plan(const int32_t* block_idx, const AttnWs& ws, const Dims& D, hipStream_t stream);
// Strided copy of n_seg runs of `words` 32-bit words (src + s * src_pitch ->
// dst + s * dst_pitch, pitches in words): moves the per-row outputs of one pass
// of a chunked call between the caller's layout and the pass's own.
hipError_t launch_copy_runs(const void* src, int64_t src_pitch, void* dst, int64_t dst_pitch, int64_t words,
                            int64_t n_seg, hipStream_t stream);
// Sorts every bin's entries of a built plan (ascending row-slot id), so that
// sums over a bin's rows run in a fixed order.
hipError_t launch_plan_sort(const AttnWs& ws, const Dims& D, hipStream_t stream);
int64_t plan_chunks(const Dims& D);       // chunk workgroups per (b, g)
int64_t plan_scan_blocks(const Dims& D);  // workgroups of the two-level scan
int64_t plan_groups(const Dims& D);       // query groups (kGroupChunks chunks) per (b, g)
int64_t plan_bins(const Dims& D);         // (b, g, query group, block) bins

// Gather plan + gathered non-local tiles + local tiles with the merge.
hipError_t launch_sparse_attn(const uint16_t* q, const void* k, const void* v, const int32_t* block_idx,
                              uint16_t* out, float* lse, const AttnWs& ws, const Dims& D, hipStream_t stream);
// The same in two parts, for callers that put the plan on another stream: the
// forward's view of D (its tiles hold 128 rows, so pt is that of 128 rows; a
// workspace sized for D fits it), and the two attention kernels over a built
// plan of that view.
Dims fwd_attn_dims(const Dims& D);
hipError_t launch_attn_kernels(const uint16_t* q, const void* k, const void* v, uint16_t* out, float* lse,
                               const AttnWs& ws, const Dims& F, hipStream_t stream);

// KL alignment of the index branch to the main branch's group-averaged
// attention over the selected tokens (needs the forward's lse); kl_part holds
// one float4 per (row, slot).  Supported for G in {4, 8, 16, 32}, bf16 index
// inputs and uniform batches.  teacher (optional): fp16 [B][H_kv][n_q][k+1][kBk],
// the teacher's weight of each key of each (row, slot) that the row uses.
bool kl_supported(const Dims& D);
hipError_t launch_index_kl(const uint16_t* q, const uint16_t* k, const uint16_t* index_q, const uint16_t* index_k,
                           const int32_t* block_idx, const float* lse, float* kl, float* lse_index, uint16_t* teacher,
                           const AttnWs& ws, float4* kl_part, const Dims& D, hipStream_t stream);

// KL backward into the index branch: d_index_q, d_index_k (bf16); diq_part
// holds one bf16 partial per (row, slot), dik_group each group's fp32 share.
// The first form forms the teacher again from q, k and lse; the second reads
// the one launch_index_kl stored.
hipError_t launch_index_kl_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* index_q, const uint16_t* index_k,
                               const int32_t* block_idx, const float* lse, const float* lse_index, const float* wrow,
                               uint16_t* d_index_q, uint16_t* d_index_k, const AttnWs& ws, uint16_t* diq_part,
                               float* dik_group, const Dims& D, hipStream_t stream);
hipError_t launch_index_kl_bwd_teacher(const uint16_t* index_q, const uint16_t* index_k, const int32_t* block_idx,
                                       const uint16_t* teacher, const float* lse_index, const float* wrow,
                                       uint16_t* d_index_q, uint16_t* d_index_k, const AttnWs& ws,
                                       uint16_t* diq_part, float* dik_group, const Dims& D, hipStream_t stream);

// Main-branch backward over the forward's selection: dq, dk, dv (bf16) from
// dout, out and lse; dq_part holds one bf16 partial per (row, slot, head),
// delta the per-(row, head) dO . O.
hipError_t launch_sparse_attn_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* block_idx,
                                  const uint16_t* out, const float* lse, const uint16_t* dout, uint16_t* dq,
                                  uint16_t* dk, uint16_t* dv, const AttnWs& ws, uint16_t* dq_part, float* delta,
                                  const Dims& D, hipStream_t stream);

// Dense mode (the indexer warmup): causal GQA attention over every visible
// token, and the KL value over every visible token (needs the dense lse).
hipError_t launch_dense_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* out, float* lse,
                             const Dims& D, hipStream_t stream);
hipError_t launch_dense_index_kl(const uint16_t* q, const uint16_t* k, const uint16_t* index_q,
                                 const uint16_t* index_k, const float* lse, float* kl, float* lse_index,
                                 const Dims& D, hipStream_t stream);

// Decode-shaped calls (few query rows per sequence).
bool use_index_small(const Dims& D);   // at most 16 (query, group) rows per sequence
bool use_attn_rows(const Dims& D);     // query-outer attention
size_t attn_rows_partial_bytes(const Dims& D);
hipError_t launch_index_small(const void* index_q, const void* index_k, float* pooled, const Dims& D,
                              hipStream_t stream);
hipError_t launch_attn_rows(const uint16_t* q, const void* k, const void* v, const int32_t* block_idx,
                            uint16_t* out, float* lse, float* part, const Dims& D, hipStream_t stream);

}  // namespace msa
