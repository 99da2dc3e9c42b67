// The C ABI of include/msa.h: argument validation, workspace layout and
// dispatch.  Every check runs on the host before any HIP call, so a rejected
// call enqueues nothing.
#include <algorithm>
#include <cmath>
#include <climits>
#include <cstddef>
#include <cstring>

#include "../../include/msa.h"
#include "launch.h"

namespace {

constexpr int kRowsMaxQForPasses = msa::kRowsMaxQ;  // decode-shaped calls (n_q <= 4) never run in passes

using msa::AttnWs;
using msa::Dims;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

// Validate a problem and derive the kernels' view of it.  limits = false skips
// the bounds of one launch (32-bit row and tile indices, grid sizes): a call
// that runs in passes checks them for each pass instead.
msa_status derive(const msa_problem* p, Dims* D, bool limits = true) {
  if (!p) return MSA_ERR_INVALID_ARGUMENT;
  if (p->batch < 1 || p->n_q < 1 || p->n_kv < 1 || p->h_q < 1 || p->h_kv < 1 || p->head_dim < 1 ||
      p->index_dim < 1 || p->block_size < 1 || p->topk < 1)
    return MSA_ERR_INVALID_ARGUMENT;
  if (p->h_q % p->h_kv != 0) return MSA_ERR_INVALID_ARGUMENT;
  if (p->q_offset < -1) return MSA_ERR_INVALID_ARGUMENT;
  const int64_t offset = p->q_offset == -1 ? (int64_t)p->n_kv - p->n_q : p->q_offset;
  if (offset < 0 || offset + p->n_q > p->n_kv) return MSA_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(p->softmax_scale)) return MSA_ERR_INVALID_ARGUMENT;
  if (p->index_dtype != MSA_DTYPE_BF16 && p->index_dtype != MSA_DTYPE_FP8_E4M3) return MSA_ERR_INVALID_ARGUMENT;
  if (p->kv_dtype != MSA_DTYPE_BF16 && p->kv_dtype != MSA_DTYPE_FP8_E4M3) return MSA_ERR_INVALID_ARGUMENT;
  const int64_t G = p->h_q / p->h_kv;
  const int64_t n_blk = ((int64_t)p->n_kv + p->block_size - 1) / p->block_size;
  // index ranges the kernels keep in 32 bits
  const int64_t rows = (int64_t)p->batch * p->h_kv * p->n_q;
  if (limits && (rows * p->topk > INT32_MAX || (int64_t)p->n_q * p->topk > INT32_MAX ||
                 (int64_t)p->n_q * p->h_kv > INT32_MAX))
    return MSA_ERR_INVALID_ARGUMENT;
  if ((int64_t)p->batch * p->h_kv * n_blk > INT32_MAX) return MSA_ERR_INVALID_ARGUMENT;
  if (p->head_dim != msa::kHeadDim || (p->index_dim != 64 && p->index_dim != 128) || p->block_size != msa::kBk ||
      p->topk > msa::kMaxTopk || G > msa::kMaxGroup)
    return MSA_ERR_UNSUPPORTED;
  int pt = 1;
  // positions per attention tile: pt * G rows fill the tile; pt <= Bk keeps a
  // local tile's positions inside one block
  while (pt * 2 * G <= msa::kTileRows && pt * 2 <= msa::kBk) pt *= 2;
  // launch-grid limits: y/z dims of 65535, 2^32 threads along x
  const int64_t n_groups = ((int64_t)p->n_q + msa::kChunkRows * msa::kGroupChunks - 1) /
                           (msa::kChunkRows * msa::kGroupChunks);
  const int64_t max_tiles = (rows * p->topk + pt - 1) / pt + (int64_t)p->batch * p->h_kv * n_groups * n_blk;
  if ((int64_t)p->batch * p->h_kv > 65535) return MSA_ERR_UNSUPPORTED;
  if (limits && (max_tiles * 256 >= (int64_t(1) << 32) || max_tiles * pt > INT32_MAX ||
                 rows * 64 >= (int64_t(1) << 32) || rows > 65535LL * 65535LL))
    return MSA_ERR_UNSUPPORTED;
  D->B = p->batch;
  D->n_q = p->n_q;
  D->n_kv = p->n_kv;
  D->h_q = p->h_q;
  D->h_kv = p->h_kv;
  D->G = (int32_t)G;
  D->d = p->head_dim;
  D->d_idx = p->index_dim;
  D->idx_eb = p->index_dtype == MSA_DTYPE_FP8_E4M3 ? 1 : 2;
  D->kv_eb = p->kv_dtype == MSA_DTYPE_FP8_E4M3 ? 1 : 2;
  D->k = p->topk;
  D->n_blk = (int32_t)n_blk;
  D->pt = pt;
  D->offset = offset;
  D->scale = p->softmax_scale;
  D->scale_log2 = (float)((double)p->softmax_scale * 1.4426950408889634);
  D->qo_lens = D->kv_lens = D->q_starts = D->pages = nullptr;
  D->pages_per_seq = D->num_pages = 0;
  D->total_q = 0;
  return MSA_OK;
}

// derive() plus the variable-length / paged description (vl may be null).
msa_status derive_v(const msa_problem* p, const msa_varlen* vl, Dims* D) {
  const msa_status st = derive(p, D);
  if (st != MSA_OK || !vl) return st;
  if ((vl->qo_lens || vl->kv_lens) && p->q_offset != -1) return MSA_ERR_INVALID_ARGUMENT;
  if (vl->q_starts && vl->total_q < 1) return MSA_ERR_INVALID_ARGUMENT;
  if (vl->page_table && (vl->num_pages < 1 || vl->pages_per_seq < D->n_blk)) return MSA_ERR_INVALID_ARGUMENT;
  if (vl->page_table && (int64_t)vl->num_pages * p->h_kv * msa::kBk > INT32_MAX) return MSA_ERR_INVALID_ARGUMENT;
  D->qo_lens = vl->qo_lens;
  D->kv_lens = vl->kv_lens;
  D->q_starts = vl->q_starts;
  D->total_q = vl->q_starts ? vl->total_q : 0;
  D->pages = vl->page_table;
  D->pages_per_seq = vl->page_table ? vl->pages_per_seq : 0;
  D->num_pages = vl->page_table ? vl->num_pages : 0;
  return MSA_OK;
}

// Carve the sparse-attention workspace out of `base` (nullptr: sizing only).
// with_o = false leaves out the partial outputs (the KL pass needs only the
// plan, whose fill also marks the partial lse of unused slots).
size_t attn_ws_layout(const Dims& D, char* base, AttnWs* ws, bool with_o = true) {
  const int64_t nbgt = msa::plan_bins(D);
  const int64_t slots = (int64_t)D.B * D.h_kv * D.n_q * D.k;
  const int64_t max_tiles = (slots + D.pt - 1) / D.pt + nbgt;
  size_t at = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + at : nullptr;
    at += round256(bytes);
    return p;
  };
  char* hist = take(sizeof(int32_t) * (int64_t)D.B * D.h_kv * D.n_blk * msa::plan_chunks(D));
  char* cnt = take(sizeof(int32_t) * nbgt);
  char* bsum = take(sizeof(int32_t) * 2 * msa::plan_scan_blocks(D));
  char* off = take(sizeof(int32_t) * (nbgt + 1));
  char* tile_off = take(sizeof(int32_t) * (nbgt + 1));
  char* list = take(sizeof(int2) * max_tiles * D.pt);
  const int64_t pslots = (int64_t)D.B * D.h_kv * D.n_q * (D.k + 1);  // + the local slot
  char* part_lse = take(sizeof(float) * pslots * D.G);
  // 12 bits per value (48 dwords per row and head) and two exponent bytes per lane pair
  char* part_o = with_o ? take(sizeof(uint32_t) * pslots * D.G * (msa::kHeadDim * 12 / 32)) : nullptr;
  char* part_ex = with_o ? take(sizeof(uint16_t) * pslots * D.G * 2) : nullptr;
  char* ctr = take(sizeof(int32_t) * msa::kWorkCounters);
  if (ws) {
    ws->hist = reinterpret_cast<int32_t*>(hist);
    ws->cnt = reinterpret_cast<int32_t*>(cnt);
    ws->bsum = reinterpret_cast<int32_t*>(bsum);
    ws->off = reinterpret_cast<int32_t*>(off);
    ws->tile_off = reinterpret_cast<int32_t*>(tile_off);
    ws->list = reinterpret_cast<int2*>(list);
    ws->part_lse = reinterpret_cast<float*>(part_lse);
    ws->part_o = reinterpret_cast<uint32_t*>(part_o);
    ws->part_ex = reinterpret_cast<uint16_t*>(part_ex);
    ws->ctr = reinterpret_cast<int32_t*>(ctr);
    ws->max_tiles = max_tiles;
    ws->n_bins = nbgt;
    ws->n_groups = (int32_t)msa::plan_groups(D);
  }
  return at;
}

// The gather plan keeps one LDS histogram bin per block (n_kv <= 2M tokens);
// the query-outer path of decode-shaped calls has no such limit.
bool attn_path_ok(const Dims& D) { return msa::use_attn_rows(D) || D.n_blk <= msa::kMaxPlanBlocks; }

size_t attn_bytes(const Dims& D) {
  return msa::use_attn_rows(D) ? round256(msa::attn_rows_partial_bytes(D)) : attn_ws_layout(D, nullptr, nullptr);
}

hipError_t run_attention(const Dims& D, const void* q, const void* k, const void* v, const int32_t* block_idx,
                         void* out, float* lse, char* ws_base, hipStream_t stream) {
  auto q16 = static_cast<const uint16_t*>(q);
  auto o16 = static_cast<uint16_t*>(out);
  if (msa::use_attn_rows(D))
    return msa::launch_attn_rows(q16, k, v, block_idx, o16, lse, reinterpret_cast<float*>(ws_base), D, stream);
  AttnWs ws;
  attn_ws_layout(D, ws_base, &ws);
  return msa::launch_sparse_attn(q16, k, v, block_idx, o16, lse, ws, D, stream);
}

hipError_t run_index(const Dims& D, const void* index_q, const void* index_k, float* pooled, hipStream_t stream) {
  return msa::use_index_small(D) ? msa::launch_index_small(index_q, index_k, pooled, D, stream)
                                 : msa::launch_index_scores(index_q, index_k, pooled, D, stream);
}

size_t pooled_bytes(const Dims& D) { return round256(sizeof(float) * (size_t)D.B * D.h_kv * D.n_q * D.n_blk); }

// The KL pass: the gather plan (without partial outputs), then one float4
// partial per (row, slot).
size_t kl_part_bytes(const Dims& D) { return round256(sizeof(float) * 4 * (size_t)D.B * D.h_kv * D.n_q * (D.k + 1)); }
size_t kl_bytes(const Dims& D) { return attn_ws_layout(D, nullptr, nullptr, false) + kl_part_bytes(D); }

// The backward pass: the plan, one bf16 dQ partial per (row, slot, head), the
// per-(row, head) dO . O.
size_t bwd_part_bytes(const Dims& D) {
  return round256(sizeof(uint16_t) * (size_t)D.B * D.h_kv * D.n_q * (D.k + 1) * D.G * msa::kHeadDim);
}
size_t bwd_delta_bytes(const Dims& D) { return round256(sizeof(float) * (size_t)D.B * D.h_q * D.n_q); }
// The backward walks keep per-row offsets within a sequence ((g G + h) n_q + i
// and i h_q + g G + h) in 32 bits.  derive()'s tile bound (rows k G 2 < 2^32)
// already implies h_q n_q < 2^31; the check keeps the walks safe should that
// bound change.
bool bwd_walk_ok(const Dims& D) { return (int64_t)D.h_q * D.n_q < INT32_MAX; }

size_t bwd_bytes(const Dims& D) {
  return attn_ws_layout(D, nullptr, nullptr, false) + bwd_part_bytes(D) + bwd_delta_bytes(D);
}

// The KL backward: the plan, one bf16 d_index_q partial per (row, slot), and
// each group's fp32 share of d_index_k.
size_t klb_part_bytes(const Dims& D) {
  return round256(sizeof(uint16_t) * (size_t)D.B * D.h_kv * D.n_q * (D.k + 1) * D.d_idx);
}
size_t klb_group_bytes(const Dims& D) { return round256(sizeof(float) * (size_t)D.B * D.h_kv * D.n_kv * D.d_idx); }
size_t klb_bytes(const Dims& D) {
  return attn_ws_layout(D, nullptr, nullptr, false) + klb_part_bytes(D) + klb_group_bytes(D);
}

msa_status hip_status(hipError_t e) { return e == hipSuccess ? MSA_OK : MSA_ERR_HIP; }

// ---- passes over query chunks of a long uniform prefill (msa_problem.chunk_rows)

int64_t chunk_rows_of(const msa_problem* p) {
  const int64_t c = p->chunk_rows > 0 ? p->chunk_rows : MSA_DEFAULT_CHUNK_ROWS;
  return std::max<int64_t>(MSA_CHUNK_ALIGN, c / MSA_CHUNK_ALIGN * MSA_CHUNK_ALIGN);
}

// Does a forward or attention call on this (limit-free) view run in passes?
// Uniform batches only; decode-shaped calls never do.
bool runs_in_passes(const msa_problem* p, const Dims& D, const msa_varlen* vl) {
  const bool varlen = vl && (vl->qo_lens || vl->kv_lens || vl->q_starts || vl->page_table);
  return !varlen && D.n_q > kRowsMaxQForPasses && D.n_q > chunk_rows_of(p);
}

// One pass: rows c0 .. c0 + rows - 1 of one sequence, as a batch of one.  A
// pass starts on a multiple of MSA_CHUNK_ALIGN, which is a whole number of the
// gather plan's query groups and local tiles, so each row's tiles, partials and
// merge are those of the single launch.
msa_status pass_dims(const msa_problem* p, const Dims& D, int64_t c0, int64_t rows, Dims* Dp) {
  msa_problem s = *p;
  s.batch = 1;
  s.n_q = (int32_t)rows;
  s.q_offset = D.offset + c0;
  s.chunk_rows = 0;
  return derive(&s, Dp, true);
}

// Visits every pass (b, c0, rows) of a chunked call in order; stops at the
// first non-OK status the visitor returns.
template <typename F>
msa_status for_each_pass(const msa_problem* p, const Dims& D, bool all_batches, F&& f) {
  const int64_t C = chunk_rows_of(p);
  for (int b = 0; b < (all_batches ? D.B : 1); ++b)
    for (int64_t c0 = 0; c0 < D.n_q; c0 += C) {
      const msa_status st = f(b, c0, std::min<int64_t>(C, D.n_q - c0));
      if (st != MSA_OK) return st;
    }
  return MSA_OK;
}

// The forward pass's own workspace: pooled scores only when scoring and top-k
// cannot run as one launch, then the attention's.
bool forward_fused(const Dims& D) { return !msa::use_index_small(D) && msa::index_topk_fusable(D); }
size_t forward_pass_bytes(const Dims& D) { return (forward_fused(D) ? 0 : pooled_bytes(D)) + attn_bytes(D); }

// Workspace of a chunked call: the largest pass, then one pass's block_idx and
// lse rows in the pass layout.
msa_status chunked_bytes(const msa_problem* p, const Dims& D, bool forward, size_t* bytes) {
  size_t most = 0;
  const msa_status st = for_each_pass(p, D, false, [&](int, int64_t c0, int64_t rows) {
    Dims Dp;
    const msa_status s = pass_dims(p, D, c0, rows, &Dp);
    if (s != MSA_OK) return s;
    if (!attn_path_ok(Dp)) return MSA_ERR_UNSUPPORTED;
    most = std::max(most, forward ? forward_pass_bytes(Dp) : attn_bytes(Dp));
    return MSA_OK;
  });
  if (st != MSA_OK) return st;
  const int64_t C = std::min<int64_t>(chunk_rows_of(p), D.n_q);
  *bytes = most + round256(sizeof(int32_t) * C * D.h_kv * D.k) + round256(sizeof(float) * C * D.h_q);
  return MSA_OK;
}

// One unchunked forward pass on view D (pointers at the view's row 0).
hipError_t forward_pass(const Dims& D, const void* q, const void* k, const void* v, const void* index_q,
                        const void* index_k, void* out, int32_t* block_idx, float* lse, char* ws, hipStream_t stream) {
  hipError_t e;
  size_t at = 0;
  if (forward_fused(D)) {
    e = msa::launch_index_topk(index_q, index_k, block_idx, D, stream);
  } else {
    float* pooled = reinterpret_cast<float*>(ws);
    at = pooled_bytes(D);
    e = run_index(D, index_q, index_k, pooled, stream);
    if (e == hipSuccess) e = msa::launch_block_topk(pooled, block_idx, D, stream);
  }
  if (e != hipSuccess) return e;
  return run_attention(D, q, k, v, block_idx, out, lse, ws + at, stream);
}

// A forward or attention call in passes.  Per pass: the inputs are the
// caller's rows c0.. of sequence b (contiguous: q, index_q, out are token
// major); block_idx and lse rows live in the pass layout at the workspace's
// tail and are copied from (attention) or to (both) the caller's
// [B][H_kv][n_q][k] and [B][H_q][n_q] tensors.
msa_status run_in_passes(const msa_problem* p, const Dims& D, bool forward, const void* q, const void* k,
                         const void* v, const void* index_q, const void* index_k, void* out, int32_t* block_idx,
                         float* lse, char* ws, hipStream_t stream) {
  size_t total = 0;
  msa_status st = chunked_bytes(p, D, forward, &total);
  if (st != MSA_OK) return st;
  const int64_t C = std::min<int64_t>(chunk_rows_of(p), D.n_q);
  char* tail = ws + total - round256(sizeof(int32_t) * C * D.h_kv * D.k) - round256(sizeof(float) * C * D.h_q);
  int32_t* bidx_p = reinterpret_cast<int32_t*>(tail);
  float* lse_p = reinterpret_cast<float*>(tail + round256(sizeof(int32_t) * C * D.h_kv * D.k));
  const char* qb = static_cast<const char*>(q);
  const char* kb = static_cast<const char*>(k);
  const char* vb = static_cast<const char*>(v);
  const char* iqb = static_cast<const char*>(index_q);
  const char* ikb = static_cast<const char*>(index_k);
  char* ob = static_cast<char*>(out);
  return for_each_pass(p, D, true, [&](int b, int64_t c0, int64_t rows) {
    Dims Dp;
    msa_status s = pass_dims(p, D, c0, rows, &Dp);
    if (s != MSA_OK) return s;
    const int64_t row0 = (int64_t)b * D.n_q + c0;                        // caller's token-major row
    const int64_t q_off = row0 * D.h_q * msa::kHeadDim * 2;              // bytes, bf16
    const int64_t kv_off = (int64_t)b * D.h_kv * D.n_kv * msa::kHeadDim * D.kv_eb;
    int32_t* bidx_dst = block_idx + ((int64_t)b * D.h_kv * D.n_q + c0) * D.k;
    float* lse_dst = lse ? lse + (int64_t)b * D.h_q * D.n_q + c0 : nullptr;
    hipError_t e;
    if (forward) {
      const int64_t iq_off = row0 * D.h_kv * D.d_idx * D.idx_eb;
      const int64_t ik_off = (int64_t)b * D.n_kv * D.d_idx * D.idx_eb;
      e = forward_pass(Dp, qb + q_off, kb + kv_off, vb + kv_off, iqb + iq_off, ikb + ik_off, ob + q_off, bidx_p,
                       lse ? lse_p : nullptr, ws, stream);
    } else {
      e = msa::launch_copy_runs(bidx_dst, (int64_t)D.n_q * D.k, bidx_p, rows * D.k, rows * D.k, D.h_kv, stream);
      if (e == hipSuccess)
        e = run_attention(Dp, qb + q_off, kb + kv_off, vb + kv_off, bidx_p, ob + q_off, lse ? lse_p : nullptr, ws,
                          stream);
    }
    if (e == hipSuccess && forward)
      e = msa::launch_copy_runs(bidx_p, rows * D.k, bidx_dst, (int64_t)D.n_q * D.k, rows * D.k, D.h_kv, stream);
    if (e == hipSuccess && lse) e = msa::launch_copy_runs(lse_p, rows, lse_dst, D.n_q, rows, D.h_q, stream);
    return hip_status(e);
  });
}

}  // namespace

// ---- timing marks (msa_forward_marked)
namespace {
struct MarkLog {
  hipEvent_t* events;
  const char** names;
  int cap, n;  // events available, events recorded
};
thread_local MarkLog* g_marks = nullptr;
}  // namespace

namespace msa {
void mark(const char* name, hipStream_t stream) {
  MarkLog* m = g_marks;
  if (!m || m->n >= m->cap) return;
  if (m->names) m->names[m->n - 1] = name;
  if (hipEventRecord(m->events[m->n], stream) == hipSuccess) ++m->n;
}
}  // namespace msa

static_assert(sizeof(msa_problem) == 64 && offsetof(msa_problem, index_dtype) == 52 &&
                  offsetof(msa_problem, kv_dtype) == 56 && offsetof(msa_problem, chunk_rows) == 60,
              "msa_problem layout is part of the ABI");

extern "C" {

msa_status msa_workspace_size(const msa_problem* p, int op, size_t* bytes) {
  if (!bytes) return MSA_ERR_INVALID_ARGUMENT;
  Dims D;
  if (op == MSA_OP_SPARSE_ATTN || op == MSA_OP_FORWARD) {
    const msa_status st0 = derive(p, &D, false);
    if (st0 != MSA_OK) return st0;
    if (runs_in_passes(p, D, nullptr)) return chunked_bytes(p, D, op == MSA_OP_FORWARD, bytes);
  }
  const msa_status st = derive(p, &D);
  if (st != MSA_OK) return st;
  switch (op) {
    case MSA_OP_INDEX_SCORES:
    case MSA_OP_BLOCK_TOPK:
      *bytes = 0;
      return MSA_OK;
    case MSA_OP_SPARSE_ATTN:
      if (!attn_path_ok(D)) return MSA_ERR_UNSUPPORTED;
      *bytes = attn_bytes(D);
      return MSA_OK;
    case MSA_OP_FORWARD:
      if (!attn_path_ok(D)) return MSA_ERR_UNSUPPORTED;
      *bytes = forward_pass_bytes(D);
      return MSA_OK;
    case MSA_OP_SPARSE_ATTN_BWD:
      if (D.n_blk > msa::kMaxPlanBlocks || D.kv_eb != 2 || !bwd_walk_ok(D)) return MSA_ERR_UNSUPPORTED;
      *bytes = bwd_bytes(D);
      return MSA_OK;
    case MSA_OP_INDEX_KL:
      if (D.n_blk > msa::kMaxPlanBlocks || !msa::kl_supported(D)) return MSA_ERR_UNSUPPORTED;
      *bytes = kl_bytes(D);
      return MSA_OK;
    case MSA_OP_INDEX_KL_BWD:
      if (D.n_blk > msa::kMaxPlanBlocks || !msa::kl_supported(D) || !bwd_walk_ok(D)) return MSA_ERR_UNSUPPORTED;
      *bytes = klb_bytes(D);
      return MSA_OK;
    default:
      return MSA_ERR_INVALID_ARGUMENT;
  }
}

msa_status msa_index_scores_v(const msa_problem* p, const msa_varlen* vl, const void* index_q, const void* index_k,
                              float* pooled, hipStream_t stream) {
  Dims D;
  const msa_status st = derive_v(p, vl, &D);
  if (st != MSA_OK) return st;
  if (!index_q || !index_k || !pooled) return MSA_ERR_INVALID_ARGUMENT;
  if (!aligned16(index_q) || !aligned16(index_k) || !aligned16(pooled)) return MSA_ERR_INVALID_ARGUMENT;
  return hip_status(run_index(D, index_q, index_k, pooled, stream));
}

msa_status msa_block_topk_v(const msa_problem* p, const msa_varlen* vl, const float* pooled, int32_t* block_idx,
                            hipStream_t stream) {
  Dims D;
  const msa_status st = derive_v(p, vl, &D);
  if (st != MSA_OK) return st;
  if (!pooled || !block_idx) return MSA_ERR_INVALID_ARGUMENT;
  if (!aligned16(pooled) || !aligned16(block_idx)) return MSA_ERR_INVALID_ARGUMENT;
  return hip_status(msa::launch_block_topk(pooled, block_idx, D, stream));
}

msa_status msa_sparse_attn_fwd_v(const msa_problem* p, const msa_varlen* vl, const void* q, const void* k,
                                 const void* v, const int32_t* block_idx, void* out, float* lse, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  Dims D;
  msa_status st = derive(p, &D, false);
  if (st != MSA_OK) return st;
  const bool passes = runs_in_passes(p, D, vl);
  if (!passes) st = derive_v(p, vl, &D);
  if (st != MSA_OK) return st;
  if (!q || !k || !v || !block_idx || !out || !workspace) return MSA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(block_idx) || !aligned16(out) ||
      !aligned16(workspace) || (lse && !aligned16(lse)))
    return MSA_ERR_INVALID_ARGUMENT;
  if (passes) {
    size_t need = 0;
    st = chunked_bytes(p, D, false, &need);
    if (st != MSA_OK) return st;
    if (need > workspace_bytes) return MSA_ERR_WORKSPACE_TOO_SMALL;
    return run_in_passes(p, D, false, q, k, v, nullptr, nullptr, out, const_cast<int32_t*>(block_idx), lse,
                         static_cast<char*>(workspace), stream);
  }
  if (!attn_path_ok(D)) return MSA_ERR_UNSUPPORTED;
  if (attn_bytes(D) > workspace_bytes) return MSA_ERR_WORKSPACE_TOO_SMALL;
  return hip_status(run_attention(D, q, k, v, block_idx, out, lse, static_cast<char*>(workspace), stream));
}

msa_status msa_forward_v(const msa_problem* p, const msa_varlen* vl, const void* q, const void* k, const void* v,
                         const void* index_q, const void* index_k, void* out, int32_t* block_idx, float* lse,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  Dims D;
  msa_status st = derive(p, &D, false);
  if (st != MSA_OK) return st;
  const bool passes = runs_in_passes(p, D, vl);
  if (!passes) st = derive_v(p, vl, &D);
  if (st != MSA_OK) return st;
  if (!q || !k || !v || !index_q || !index_k || !out || !block_idx || !workspace) return MSA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(index_q) || !aligned16(index_k) ||
      !aligned16(out) || !aligned16(block_idx) || !aligned16(workspace) || (lse && !aligned16(lse)))
    return MSA_ERR_INVALID_ARGUMENT;
  if (passes) {
    size_t need = 0;
    st = chunked_bytes(p, D, true, &need);
    if (st != MSA_OK) return st;
    if (need > workspace_bytes) return MSA_ERR_WORKSPACE_TOO_SMALL;
    return run_in_passes(p, D, true, q, k, v, index_q, index_k, out, block_idx, lse, static_cast<char*>(workspace),
                         stream);
  }
  if (!attn_path_ok(D)) return MSA_ERR_UNSUPPORTED;
  if (forward_pass_bytes(D) > workspace_bytes) return MSA_ERR_WORKSPACE_TOO_SMALL;
  return hip_status(forward_pass(D, q, k, v, index_q, index_k, out, block_idx, lse, static_cast<char*>(workspace),
                                 stream));
}

msa_status msa_forward_marked(const msa_problem* p, const msa_varlen* vl, const void* q, const void* k, const void* v,
                              const void* index_q, const void* index_k, void* out, int32_t* block_idx, float* lse,
                              void* workspace, size_t workspace_bytes, hipStream_t stream, hipEvent_t* events,
                              int max_events, const char** names, int* n_events) {
  if (!events || max_events < 1 || !n_events) return MSA_ERR_INVALID_ARGUMENT;
  *n_events = 0;
  {
    // validate first, so that a rejected call records nothing
    Dims D;
    const msa_status st = derive(p, &D, false);
    if (st != MSA_OK) return st;
  }
  if (hipEventRecord(events[0], stream) != hipSuccess) return MSA_ERR_HIP;
  MarkLog log{events, names, max_events, 1};
  g_marks = &log;
  const msa_status st = msa_forward_v(p, vl, q, k, v, index_q, index_k, out, block_idx, lse, workspace,
                                      workspace_bytes, stream);
  g_marks = nullptr;
  *n_events = log.n;
  return st;
}

msa_status msa_index_kl(const msa_problem* p, const void* q, const void* k, const void* index_q, const void* index_k,
                        const int32_t* block_idx, const float* lse, float* kl, float* lse_index, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  Dims D;
  const msa_status st = derive(p, &D);
  if (st != MSA_OK) return st;
  if (!q || !k || !index_q || !index_k || !block_idx || !lse || !kl || !workspace) return MSA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k) || !aligned16(index_q) || !aligned16(index_k) || !aligned16(block_idx) ||
      !aligned16(lse) || !aligned16(kl) || !aligned16(workspace) || (lse_index && !aligned16(lse_index)))
    return MSA_ERR_INVALID_ARGUMENT;
  if (D.n_blk > msa::kMaxPlanBlocks || !msa::kl_supported(D)) return MSA_ERR_UNSUPPORTED;
  if (kl_bytes(D) > workspace_bytes) return MSA_ERR_WORKSPACE_TOO_SMALL;
  AttnWs ws;
  char* base = static_cast<char*>(workspace);
  const size_t plan = attn_ws_layout(D, base, &ws, false);
  return hip_status(msa::launch_index_kl(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                         static_cast<const uint16_t*>(index_q), static_cast<const uint16_t*>(index_k),
                                         block_idx, lse, kl, lse_index, nullptr, ws,
                                         reinterpret_cast<float4*>(base + plan), D, stream));
}

msa_status msa_index_kl_teacher(const msa_problem* p, const void* q, const void* k, const void* index_q,
                                const void* index_k, const int32_t* block_idx, const float* lse, float* kl,
                                float* lse_index, void* teacher, void* workspace, size_t workspace_bytes,
                                hipStream_t stream) {
  Dims D;
  const msa_status st = derive(p, &D);
  if (st != MSA_OK) return st;
  if (!q || !k || !index_q || !index_k || !block_idx || !lse || !kl || !lse_index || !teacher || !workspace)
    return MSA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k) || !aligned16(index_q) || !aligned16(index_k) || !aligned16(block_idx) ||
      !aligned16(lse) || !aligned16(kl) || !aligned16(lse_index) || !aligned16(teacher) || !aligned16(workspace))
    return MSA_ERR_INVALID_ARGUMENT;
  if (D.n_blk > msa::kMaxPlanBlocks || !msa::kl_supported(D)) return MSA_ERR_UNSUPPORTED;
  if (kl_bytes(D) > workspace_bytes) return MSA_ERR_WORKSPACE_TOO_SMALL;
  AttnWs ws;
  char* base = static_cast<char*>(workspace);
  const size_t plan = attn_ws_layout(D, base, &ws, false);
  return hip_status(msa::launch_index_kl(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                         static_cast<const uint16_t*>(index_q), static_cast<const uint16_t*>(index_k),
                                         block_idx, lse, kl, lse_index, static_cast<uint16_t*>(teacher), ws,
                                         reinterpret_cast<float4*>(base + plan), D, stream));
}

msa_status msa_index_kl_bwd(const msa_problem* p, const void* q, const void* k, const void* index_q,
                            const void* index_k, const int32_t* block_idx, const float* lse, const float* lse_index,
                            const float* dkl, void* d_index_q, void* d_index_k, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  Dims D;
  const msa_status st = derive(p, &D);
  if (st != MSA_OK) return st;
  if (!q || !k || !index_q || !index_k || !block_idx || !lse || !lse_index || !d_index_q || !d_index_k || !workspace)
    return MSA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k) || !aligned16(index_q) || !aligned16(index_k) || !aligned16(block_idx) ||
      !aligned16(lse) || !aligned16(lse_index) || (dkl && !aligned16(dkl)) || !aligned16(d_index_q) ||
      !aligned16(d_index_k) || !aligned16(workspace))
    return MSA_ERR_INVALID_ARGUMENT;
  if (D.n_blk > msa::kMaxPlanBlocks || !msa::kl_supported(D) || !bwd_walk_ok(D)) return MSA_ERR_UNSUPPORTED;
  if (klb_bytes(D) > workspace_bytes) return MSA_ERR_WORKSPACE_TOO_SMALL;
  AttnWs ws;
  char* base = static_cast<char*>(workspace);
  const size_t plan = attn_ws_layout(D, base, &ws, false);
  auto part = reinterpret_cast<uint16_t*>(base + plan);
  auto group = reinterpret_cast<float*>(base + plan + klb_part_bytes(D));
  return hip_status(msa::launch_index_kl_bwd(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(index_q),
      static_cast<const uint16_t*>(index_k), block_idx, lse, lse_index, dkl, static_cast<uint16_t*>(d_index_q),
      static_cast<uint16_t*>(d_index_k), ws, part, group, D, stream));
}

msa_status msa_index_kl_bwd_teacher(const msa_problem* p, const void* index_q, const void* index_k,
                                    const int32_t* block_idx, const void* teacher, const float* lse_index,
                                    const float* dkl, void* d_index_q, void* d_index_k, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
  Dims D;
  const msa_status st = derive(p, &D);
  if (st != MSA_OK) return st;
  if (!index_q || !index_k || !block_idx || !teacher || !lse_index || !d_index_q || !d_index_k || !workspace)
    return MSA_ERR_INVALID_ARGUMENT;
  if (!aligned16(index_q) || !aligned16(index_k) || !aligned16(block_idx) || !aligned16(teacher) ||
      !aligned16(lse_index) || (dkl && !aligned16(dkl)) || !aligned16(d_index_q) || !aligned16(d_index_k) ||
      !aligned16(workspace))
    return MSA_ERR_INVALID_ARGUMENT;
  if (D.n_blk > msa::kMaxPlanBlocks || !msa::kl_supported(D) || !bwd_walk_ok(D)) return MSA_ERR_UNSUPPORTED;
  if (klb_bytes(D) > workspace_bytes) return MSA_ERR_WORKSPACE_TOO_SMALL;
  AttnWs ws;
  char* base = static_cast<char*>(workspace);
  const size_t plan = attn_ws_layout(D, base, &ws, false);
  auto part = reinterpret_cast<uint16_t*>(base + plan);
  auto group = reinterpret_cast<float*>(base + plan + klb_part_bytes(D));
  return hip_status(msa::launch_index_kl_bwd_teacher(
      static_cast<const uint16_t*>(index_q), static_cast<const uint16_t*>(index_k), block_idx,
      static_cast<const uint16_t*>(teacher), lse_index, dkl, static_cast<uint16_t*>(d_index_q),
      static_cast<uint16_t*>(d_index_k), ws, part, group, D, stream));
}

msa_status msa_sparse_attn_bwd(const msa_problem* p, const void* q, const void* k, const void* v,
                               const int32_t* block_idx, const void* out, const float* lse, const void* dout, void* dq,
                               void* dk, void* dv, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  Dims D;
  const msa_status st = derive(p, &D);
  if (st != MSA_OK) return st;
  if (!q || !k || !v || !block_idx || !out || !lse || !dout || !dq || !dk || !dv || !workspace)
    return MSA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(block_idx) || !aligned16(out) ||
      !aligned16(lse) || !aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) ||
      !aligned16(workspace))
    return MSA_ERR_INVALID_ARGUMENT;
  if (D.n_blk > msa::kMaxPlanBlocks || D.kv_eb != 2 || !bwd_walk_ok(D)) return MSA_ERR_UNSUPPORTED;
  if (bwd_bytes(D) > workspace_bytes) return MSA_ERR_WORKSPACE_TOO_SMALL;
  AttnWs ws;
  char* base = static_cast<char*>(workspace);
  const size_t plan = attn_ws_layout(D, base, &ws, false);
  auto part = reinterpret_cast<uint16_t*>(base + plan);
  auto delta = reinterpret_cast<float*>(base + plan + bwd_part_bytes(D));
  return hip_status(msa::launch_sparse_attn_bwd(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), block_idx,
      static_cast<const uint16_t*>(out), lse, static_cast<const uint16_t*>(dout), static_cast<uint16_t*>(dq),
      static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv), ws, part, delta, D, stream));
}

msa_status msa_dense_attn_fwd(const msa_problem* p, const void* q, const void* k, const void* v, void* out, float* lse,
                              hipStream_t stream) {
  Dims D;
  const msa_status st = derive(p, &D);
  if (st != MSA_OK) return st;
  if (!q || !k || !v || !out) return MSA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || (lse && !aligned16(lse)))
    return MSA_ERR_INVALID_ARGUMENT;
  if (D.kv_eb != 2) return MSA_ERR_UNSUPPORTED;
  return hip_status(msa::launch_dense_attn(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                           static_cast<const uint16_t*>(v), static_cast<uint16_t*>(out), lse, D,
                                           stream));
}

msa_status msa_dense_index_kl(const msa_problem* p, const void* q, const void* k, const void* index_q,
                              const void* index_k, const float* lse, float* kl, float* lse_index, hipStream_t stream) {
  Dims D;
  const msa_status st = derive(p, &D);
  if (st != MSA_OK) return st;
  if (!q || !k || !index_q || !index_k || !lse || !kl) return MSA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k) || !aligned16(index_q) || !aligned16(index_k) || !aligned16(lse) ||
      !aligned16(kl) || (lse_index && !aligned16(lse_index)))
    return MSA_ERR_INVALID_ARGUMENT;
  if (!msa::kl_supported(D)) return MSA_ERR_UNSUPPORTED;
  return hip_status(msa::launch_dense_index_kl(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                               static_cast<const uint16_t*>(index_q),
                                               static_cast<const uint16_t*>(index_k), lse, kl, lse_index, D, stream));
}

msa_status msa_index_scores(const msa_problem* p, const void* index_q, const void* index_k, float* pooled,
                            hipStream_t stream) {
  return msa_index_scores_v(p, nullptr, index_q, index_k, pooled, stream);
}

msa_status msa_block_topk(const msa_problem* p, const float* pooled, int32_t* block_idx, hipStream_t stream) {
  return msa_block_topk_v(p, nullptr, pooled, block_idx, stream);
}

msa_status msa_sparse_attn_fwd(const msa_problem* p, const void* q, const void* k, const void* v,
                               const int32_t* block_idx, void* out, float* lse, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
  return msa_sparse_attn_fwd_v(p, nullptr, q, k, v, block_idx, out, lse, workspace, workspace_bytes, stream);
}

msa_status msa_forward(const msa_problem* p, const void* q, const void* k, const void* v, const void* index_q,
                       const void* index_k, void* out, int32_t* block_idx, float* lse, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  return msa_forward_v(p, nullptr, q, k, v, index_q, index_k, out, block_idx, lse, workspace, workspace_bytes,
                       stream);
}

const char* msa_status_string(msa_status s) {
  switch (s) {
    case MSA_OK:
      return "ok";
    case MSA_ERR_INVALID_ARGUMENT:
      return "invalid argument";
    case MSA_ERR_UNSUPPORTED:
      return "unsupported configuration";
    case MSA_ERR_WORKSPACE_TOO_SMALL:
      return "workspace too small";
    case MSA_ERR_HIP:
      return "HIP launch failure";
  }
  return "unknown status";
}

}  // extern "C"
