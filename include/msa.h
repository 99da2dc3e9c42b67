/*
 * msa.h -- C ABI of MiniMax Sparse Attention (MSA) for AMD Instinct MI355X
 * (gfx950): the forward pass (index scores, block top-k, sparse attention),
 * variable-length and paged batches, FP8 index inputs and K/V caches, and the
 * training-side calls (the KL alignment value and its gradient, the sparse
 * attention backward, dense mode for the indexer warmup).
 *
 * The method (page "MiniMax 发布 MSA 稀疏注意力方法，开源推理内核并推出 MiniMax-M3
 * 模型", sections 什么是 MSA and 两个分支如何工作): an Index Branch scores every
 * causally visible key with one index-query head per GQA group against one
 * shared index-key head, max-pools the scores to blocks of Bk tokens and keeps
 * the top-k blocks per query and group, the query's own (local) block always
 * taking one slot; a Main Branch then runs exact scaled dot-product softmax
 * attention, per query head, over the causally visible tokens of its group's
 * selected blocks.  The same page's "运行 Kernel" section shows the three calls
 * of the released library (a max-score proxy pass, sparse_topk_select, a
 * sparse attention pass); the entry points below follow that split.
 *
 * Notation: B batch, n_q query rows per call, n_kv key/value tokens,
 * H_q query heads, H_kv key/value heads (= GQA groups), G = H_q / H_kv,
 * d head dim, d_idx index dim, Bk block size, k blocks kept,
 * n_blk = ceil(n_kv / Bk).  Query row i sits at position p_i = q_offset + i,
 * its local block is l_i = floor(p_i / Bk), key j is visible to it iff
 * j <= p_i.  Query head h belongs to group g = floor(h / G).
 *
 * Tensor layouts (all dense, row-major, contiguous):
 *   q, out     [B][n_q][H_q][d]        bf16
 *   k, v       [B][H_kv][n_kv][d]      bf16 or FP8 E4M3  (each 128-token block of one head
 *                                             is one contiguous 32 KiB run)
 *   index_q    [B][n_q][H_kv][d_idx]   bf16 or FP8 E4M3 (one index-query head per group)
 *   index_k    [B][n_kv][d_idx]        bf16 or FP8 E4M3 (one shared index-key head)
 *   pooled     [B][H_kv][n_q][n_blk]   fp32
 *   block_idx  [B][H_kv][n_q][k]       int32
 *   lse        [B][H_q][n_q]           fp32, natural log (optional output)
 *
 * Ownership and execution: the caller owns every buffer (device memory) and
 * the workspace.  The library allocates no device memory, keeps no state
 * between calls and may be called concurrently on different streams with
 * different workspaces.  Each call validates its arguments on the host, then
 * only enqueues kernels on `stream` and returns; results are valid once the
 * stream has been synchronised.
 *
 * Errors: argument checks run before any HIP call.  On failure nothing is
 * enqueued and the call returns MSA_ERR_INVALID_ARGUMENT (bad shapes, null or
 * misaligned pointers, q_offset + n_q > n_kv, k < 1, H_q % H_kv != 0, index
 * overflow, an unknown index_dtype or kv_dtype) or MSA_ERR_UNSUPPORTED (shapes
 * the kernels are not built for: d != 128, d_idx not in {64, 128}, Bk != 128,
 * k > 64, G > 128; the further limits of each call are stated with it).  A failed
 * kernel launch returns MSA_ERR_HIP.  No C++ exception crosses the ABI.
 * All device pointers must be 16-byte aligned; NaN inputs are not supported.
 */
#ifndef MSA_H_
#define MSA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MSA_OK = 0,
  MSA_ERR_INVALID_ARGUMENT = 1,
  MSA_ERR_UNSUPPORTED = 2,
  MSA_ERR_WORKSPACE_TOO_SMALL = 3,
  MSA_ERR_HIP = 4
} msa_status;

/* Element type of index_q and index_k.  The released kernels take FP8 as
 * well as BF16 (page "MiniMax lança MSA…", section "Kernel open source e
 * MiniMax-M3"); the 8-bit format is OCP E4M3 (bias 7, largest finite value
 * 448, no infinities, NaN = all exponent and mantissa bits set).  Index scores
 * are then the raw dot products of the E4M3 values, exact products accumulated
 * in fp32; a per-tensor quantisation scale is a positive factor that leaves
 * the selection unchanged and is the caller's to apply.
 *
 * K and V may be FP8 E4M3 as well (kv_dtype): the main branch then attends over
 * the values the codes represent, each widened exactly to bf16 as it is staged,
 * so the arithmetic after the load is the bf16 path's.  No scale is applied: a
 * per-tensor K scale folds into softmax_scale, a V scale multiplies the output
 * and is the caller's.  FP8 K/V is taken by msa_sparse_attn_fwd and
 * msa_forward (and their _v forms); the KL, dense and backward calls return
 * MSA_ERR_UNSUPPORTED for it.  q and out stay bf16. */
typedef enum {
  MSA_DTYPE_BF16 = 0,
  MSA_DTYPE_FP8_E4M3 = 1
} msa_dtype;

/* One problem instance.  q_offset = -1 means bottom-right alignment,
 * q_offset = n_kv - n_q (prefill: n_q = n_kv gives 0; decode: n_q = 1 puts the
 * query on the last cached token, whose block is its local block).
 * index_dtype and kv_dtype are msa_dtypes (0, bf16, when the struct is
 * zero-initialised).
 *
 * chunk_rows bounds the workspace of a long prefill: msa_forward and
 * msa_sparse_attn_fwd on a uniform batch (no msa_varlen) whose n_q exceeds it
 * run as successive passes over chunk_rows query rows of one sequence, and
 * their workspace holds one pass (the per-(row, slot) partial outputs grow
 * with the rows of a pass, not with n_q).  0 means the library's default,
 * MSA_DEFAULT_CHUNK_ROWS; other values are rounded down to a multiple of
 * MSA_CHUNK_ALIGN (at least one).  Each row's results do not depend on the
 * chunking: a chunked call writes the same bits as one pass. */
typedef struct {
  int32_t batch, n_q, n_kv;
  int32_t h_q, h_kv;
  int32_t head_dim, index_dim;
  int32_t block_size, topk;
  int64_t q_offset;
  float softmax_scale; /* 1/sqrt(d) in the standard configuration */
  int32_t index_dtype; /* element type of index_q and index_k */
  int32_t kv_dtype;    /* element type of k and v (and of k_pages, v_pages) */
  int32_t chunk_rows;  /* query rows per pass of a long prefill (0: MSA_DEFAULT_CHUNK_ROWS) */
} msa_problem;

#define MSA_DEFAULT_CHUNK_ROWS 131072
#define MSA_CHUNK_ALIGN 8192

/* Which call a workspace is sized for. */
typedef enum {
  MSA_OP_INDEX_SCORES = 0,
  MSA_OP_BLOCK_TOPK = 1,
  MSA_OP_SPARSE_ATTN = 2,
  MSA_OP_FORWARD = 3,
  MSA_OP_INDEX_KL = 4,
  MSA_OP_SPARSE_ATTN_BWD = 5,
  MSA_OP_INDEX_KL_BWD = 6
} msa_op;

/* Bytes of device workspace the call `op` needs for problem `p` (0 for the
 * calls that take none).  Host only; enqueues nothing.
 *
 * How the forward workspace grows (uniform batch, G = 8, k = 16, d = 128):
 * the attention's partial outputs take (k + 1) * G * (3 d / 2 + 8) bytes (a
 * 12-bit code per value, a scale exponent byte per 32 values and an fp32 lse
 * per head) plus a few plan bytes per (sequence, group, query row) of one
 * pass, about 214 KiB per query position at H_kv = 8, so at most ~29 GB for a pass of
 * MSA_DEFAULT_CHUNK_ROWS rows whatever n_q is (a 1M-token prefill fits one
 * MI355X); the fp32 pooled scores [B][H_kv][rows][n_blk] are added only when
 * scoring and top-k cannot run as one launch (few rows against a long cache,
 * e.g. a chunk of 8192 rows at a 1M-token cache).  Decode-shaped calls (n_q
 * <= 4) need a few MiB.  A smaller chunk_rows trades passes for workspace. */
msa_status msa_workspace_size(const msa_problem* p, int op, size_t* bytes);

/*
 * Index Branch, scoring and block max-pool (section 两个分支如何工作: score the
 * visible keys with the group's index-query head against the shared index-key
 * head, then max-pool to blocks; reading R1: the score is the raw dot product).
 *   pooled[b][g][i][t] = max_{j in block t, j <= p_i} sum_c index_q[b][i][g][c] * index_k[b][j][c]
 * for t = 0 .. l_i, computed with fp32 accumulation of exact bf16 (or E4M3)
 * products.
 * Entries with t > l_i are not written (their contents are unspecified).
 */
msa_status msa_index_scores(const msa_problem* p, const void* index_q, const void* index_k, float* pooled,
                            hipStream_t stream);

/*
 * Index Branch, exp-free block top-k (section 两个分支如何工作: top-k per query
 * and group with the local block always included; section 内核协同设计: softmax
 * keeps the order, so the raw pooled scores are ranked directly).
 *   block_idx[b][g][i][:] = { l_i } U top_(k-1) of { 0 .. l_i - 1 } by
 *   (pooled desc, block index asc), written in ascending order; when
 *   l_i + 1 <= k every visible block is kept and the tail is -1.
 * Equal scores (including -0 vs +0) go to the lower block index; the result is
 * a deterministic function of the fp32 input.
 */
msa_status msa_block_topk(const msa_problem* p, const float* pooled, int32_t* block_idx, hipStream_t stream);

/*
 * Main Branch on a given block set (section 两个分支如何工作: gather the causally
 * visible tokens of the selected blocks and run scaled dot-product softmax per
 * query head, the group's block set shared by its heads; section 内核协同设计:
 * KV-outer iteration with gathered queries and a separate merge stage).
 *   out[b][i][h] = sum_{j in T} softmax_j(scale * q[b][i][h] . k[b][g][j]) v[b][g][j],
 *   T = { j <= p_i : floor(j / Bk) in S }, S = the valid entries of
 *   block_idx[b][g][i] together with l_i.
 * Each block_idx row must be ascending with entries in [0, l_i] followed by -1
 * padding (as msa_block_topk writes it); the local block l_i is always
 * attended, listed or not.  out is bf16 (rounded to nearest even from fp32);
 * lse (nullable) gets ln sum_{j in T} exp(scale * q . k_j).  Scores and
 * sums are fp32; the probabilities enter P V as bf16, and on the local block
 * as two bf16 parts (16 significant bits), so a row whose weight sits on its
 * few visible local keys keeps its accuracy.  With kv_dtype FP8 E4M3 the K and
 * V codes are widened exactly to bf16 as they are loaded.
 * Needs workspace of msa_workspace_size(p, MSA_OP_SPARSE_ATTN).
 */
msa_status msa_sparse_attn_fwd(const msa_problem* p, const void* q, const void* k, const void* v,
                               const int32_t* block_idx, void* out, float* lse, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);

/*
 * The whole forward pass: index scores, block top-k, sparse attention.
 * Writes out, block_idx and (when non-null) lse exactly as the three calls
 * above would.  Needs workspace of msa_workspace_size(p, MSA_OP_FORWARD).
 */
msa_status msa_forward(const msa_problem* p, const void* q, const void* k, const void* v, const void* index_q,
                       const void* index_k, void* out, int32_t* block_idx, float* lse, void* workspace,
                       size_t workspace_bytes, hipStream_t stream);

/*
 * KL alignment of the Index Branch to the Main Branch: the forward value of
 * the loss that trains the index projections (section MSA 如何训练: top-k has no
 * gradient, so the Index Branch's distribution is matched to the Main
 * Branch's; the teacher is the Main Branch's distribution over the selected
 * tokens averaged over the group's heads).  For every (b, g, i), over
 * T = { j <= p_i : floor(j / Bk) in S } as in msa_sparse_attn_fwd:
 *   teacher  t_j = (1/G) sum_{h in g} exp(scale * q[b][i][h] . k[b][g][j] - lse[b][h][i]),
 *   student  s_j = softmax_{j in T}(index_q[b][i][g] . index_k[b][j])   (raw index scores),
 *   kl[b][g][i] = sum_{j in T} t_j ln(t_j / s_j)   (fp32; terms with t_j = 0 add 0);
 *   lse_index[b][g][i] (nullable) = ln sum_{j in T} exp(index_q . index_k_j), the
 *   student's log-normaliser, which msa_index_kl_bwd takes.
 * lse is the natural-log output of msa_sparse_attn_fwd (or msa_forward) for
 * the same block_idx; the teacher is normalised by it, so its weights sum to 1
 * to within that lse's accuracy.  kl is [B][H_kv][n_q] fp32.  Supported for
 * G in {4, 8, 16, 32}, bf16 index inputs, bf16 K/V and uniform batches (else
 * MSA_ERR_UNSUPPORTED).  Needs workspace of msa_workspace_size(p,
 * MSA_OP_INDEX_KL).  The training reduction (mean over rows, the loss weight)
 * and the gradient are the caller's.
 */
msa_status msa_index_kl(const msa_problem* p, const void* q, const void* k, const void* index_q, const void* index_k,
                        const int32_t* block_idx, const float* lse, float* kl, float* lse_index, void* workspace,
                        size_t workspace_bytes, hipStream_t stream);

/*
 * Backward of msa_index_kl into the Index Branch (section MSA 如何训练: the KL
 * loss trains only the index projections; gradient detach keeps it off the
 * backbone, so the teacher is a constant here and q, k get no gradient).
 * With z_j = index_q[b][i][g] . index_k[b][j], s_j = exp(z_j - lse_index[b][g][i])
 * and t_j the teacher of msa_index_kl, over the same T:
 *   g_j = dkl[b][g][i] * (s_j - t_j)      (dkl = dL/dkl; NULL means all ones),
 *   d_index_q[b][i][g] = sum_{j in T} g_j index_k[b][j],
 *   d_index_k[b][j]    = sum over every (g, i) with j in its T of g_j index_q[b][i][g].
 * lse and lse_index are msa_sparse_attn_fwd's and msa_index_kl's outputs for
 * the same block_idx.  d_index_q and d_index_k have index_q's and index_k's
 * layouts (bf16, overwritten; keys no row reaches get 0).  Same support as
 * msa_index_kl; needs workspace of msa_workspace_size(p, MSA_OP_INDEX_KL_BWD).
 * Reduced without atomics (one workgroup per (sequence, group, block), then
 * the groups in order) over rows in a fixed order (sorted plan bins), so the
 * result is bitwise reproducible.
 */
msa_status msa_index_kl_bwd(const msa_problem* p, const void* q, const void* k, const void* index_q,
                            const void* index_k, const int32_t* block_idx, const float* lse, const float* lse_index,
                            const float* dkl, void* d_index_q, void* d_index_k, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/*
 * msa_index_kl, and the teacher kept for the backward: teacher (fp16,
 * [B][H_kv][n_q][k+1][Bk], caller-allocated, MSA_TEACHER_BYTES(p) bytes)
 * receives t_j of every key of every block a row uses: element
 * [b][g][i][s][j % Bk] for the block in slot s of block_idx[b][g][i] (s = k:
 * the local block), 0 for keys outside T.  Entries of slots the row does not
 * use (-1, or the local block listed again) are left as they were.  lse_index
 * is required here.  Same support and workspace as msa_index_kl; kl and
 * lse_index are the values msa_index_kl writes.
 */
#define MSA_TEACHER_BYTES(p) \
  ((size_t)(p)->batch * (p)->h_kv * (p)->n_q * ((p)->topk + 1) * (p)->block_size * 2)
msa_status msa_index_kl_teacher(const msa_problem* p, const void* q, const void* k, const void* index_q,
                                const void* index_k, const int32_t* block_idx, const float* lse, float* kl,
                                float* lse_index, void* teacher, void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

/*
 * msa_index_kl_bwd from the teacher msa_index_kl_teacher kept (for the same
 * block_idx, and with its lse_index): the same g_j, d_index_q and d_index_k
 * with t_j read instead of formed from q, k and lse, so no Main Branch input
 * is read.  t_j enters as the fp16 value stored (relative error 2^-11).  Same
 * support, workspace (MSA_OP_INDEX_KL_BWD) and reproducibility as
 * msa_index_kl_bwd.
 */
msa_status msa_index_kl_bwd_teacher(const msa_problem* p, const void* index_q, const void* index_k,
                                    const int32_t* block_idx, const void* teacher, const float* lse_index,
                                    const float* dkl, void* d_index_q, void* d_index_k, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream);

/*
 * Backward of msa_sparse_attn_fwd: the gradients the language-model loss sends
 * into the Main Branch (section MSA 如何训练), over the same token sets T as
 * the forward (block_idx as the forward used it, the local block always in).
 * With dout = dL/dout, for every (b, i, h) of group g and j in T:
 *   P_j = exp(scale q . k_j - lse),  Delta = dout . out,
 *   dS_j = P_j (dout . v_j - Delta),
 *   dq[b][i][h] = scale sum_j dS_j k_j,
 *   dk[b][g][j] = scale sum over rows and heads of dS_j q,
 *   dv[b][g][j] = sum over rows and heads of P_j dout.
 * out and lse are the forward's outputs for the same inputs; dq has q's layout,
 * dk and dv k's (bf16, overwritten; keys no row attends get 0).  Needs
 * workspace of msa_workspace_size(p, MSA_OP_SPARSE_ATTN_BWD); uniform batches and bf16
 * K/V (else MSA_ERR_UNSUPPORTED).
 * dk and dv are reduced without atomics (one workgroup owns each block) over
 * rows in a fixed order (the gather plan's bins are sorted by row and slot
 * first), so the result is bitwise reproducible.
 */
msa_status msa_sparse_attn_bwd(const msa_problem* p, const void* q, const void* k, const void* v,
                               const int32_t* block_idx, const void* out, const float* lse, const void* dout, void* dq,
                               void* dk, void* dv, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Dense mode: both branches over every visible token, as during the indexer
 * warmup (section MSA 如何训练: in the first iterations both branches run full
 * attention, so that the indexer learns from the KL loss before it routes).
 *
 * msa_dense_attn_fwd: causal GQA attention, out[b][i][h] = sum_{j <= p_i}
 * softmax_j(scale * q . k[b][g][j]) v[b][g][j], with lse (nullable) the natural
 * log-sum-exp; layouts as for msa_sparse_attn_fwd.  No workspace.
 *
 * msa_dense_index_kl: the KL value (and lse_index) of msa_index_kl with
 * T = { j <= p_i }; lse is msa_dense_attn_fwd's.  Same support as msa_index_kl (G in {4, 8, 16,
 * 32}, bf16 index inputs).  No workspace.
 *
 * Both take uniform batches (no msa_varlen form) and bf16 K/V (FP8 K/V:
 * MSA_ERR_UNSUPPORTED).
 */
msa_status msa_dense_attn_fwd(const msa_problem* p, const void* q, const void* k, const void* v, void* out, float* lse,
                              hipStream_t stream);
msa_status msa_dense_index_kl(const msa_problem* p, const void* q, const void* k, const void* index_q,
                              const void* index_k, const float* lse, float* kl, float* lse_index, hipStream_t stream);

/*
 * Variable-length batches and paged caches (section 运行 Kernel: the kernels
 * take per-sequence query and cache lengths and K/V held in pages of
 * block_size tokens addressed through a page table).  All pointers are device
 * memory; each may be NULL on its own, meaning the uniform case:
 *   qo_lens[b]    query rows of sequence b (NULL: p->n_q each);
 *   kv_lens[b]    cached tokens of sequence b (NULL: p->n_kv each);
 *   q_starts[b]   first row of sequence b in the packed q, index_q and out,
 *                 which then hold total_q rows (NULL: row b * n_q + i);
 *   page_table    [batch][pages_per_seq]: the physical page holding logical
 *                 block t of sequence b (NULL: contiguous caches).
 * With qo_lens or kv_lens given, p->q_offset must be -1 and the queries of a
 * sequence sit at the end of its cache: p_i = kv_len - qo_len + i; p->n_q and
 * p->n_kv are the maxima (qo_len <= n_q, kv_len <= n_kv, qo_len <= kv_len) and
 * size the launches and the workspace.  Per-row outputs (pooled, block_idx,
 * lse) keep p->n_q rows per (sequence, group or head); rows i >= qo_len are
 * left untouched.  With a page table, k and v are page pools
 * [num_pages][h_kv][block_size][head_dim] and index_k is
 * [num_pages][block_size][index_dim]; pages_per_seq >= ceil(n_kv / block_size).
 * Lengths above the maxima, starts past total_q and page ids outside the pool
 * are clamped (wrong results for that sequence, but no access outside the
 * buffers).  The calls below equal the plain calls when vl is NULL.
 */
typedef struct {
  const int32_t* qo_lens;
  const int32_t* kv_lens;
  const int32_t* q_starts;
  int32_t total_q;
  const int32_t* page_table;
  int32_t pages_per_seq;
  int32_t num_pages;
} msa_varlen;

msa_status msa_index_scores_v(const msa_problem* p, const msa_varlen* vl, const void* index_q, const void* index_k,
                              float* pooled, hipStream_t stream);
msa_status msa_block_topk_v(const msa_problem* p, const msa_varlen* vl, const float* pooled, int32_t* block_idx,
                            hipStream_t stream);
msa_status msa_sparse_attn_fwd_v(const msa_problem* p, const msa_varlen* vl, const void* q, const void* k,
                                 const void* v, const int32_t* block_idx, void* out, float* lse, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);
msa_status msa_forward_v(const msa_problem* p, const msa_varlen* vl, const void* q, const void* k, const void* v,
                         const void* index_q, const void* index_k, void* out, int32_t* block_idx, float* lse,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * msa_forward without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  The workspace is a fixed array of
 * MSA_NOALLOC_SCRATCH_BYTES in the library's own device memory, one per GPU,
 * held until the process ends; the call allocates nothing.  Problems whose
 * msa_workspace_size(p, MSA_OP_FORWARD) exceeds it return
 * MSA_ERR_WORKSPACE_TOO_SMALL with nothing enqueued (it covers decode steps
 * such as 64 sequences against 256K-token caches, and prefills of a few
 * thousand rows; use msa_forward with a caller's workspace beyond that).
 * Results equal msa_forward's bit for bit.  All calls on one GPU share its
 * array: calls that overlap in time on one GPU race and must be serialised
 * by the caller (one stream, or events).  Other arguments and errors as
 * msa_forward.
 */
#define MSA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
msa_status msa_forward_noalloc(const msa_problem* p, const void* q, const void* k, const void* v,
                               const void* index_q, const void* index_k, void* out, int32_t* block_idx, float* lse,
                               hipStream_t stream);

/*
 * msa_forward_v with timing marks, for benchmarks: the per-kernel times of one
 * forward pass, taken on the launch stream.  events[0] is recorded on `stream`
 * before the call's first kernel, events[i] right after its i-th kernel
 * launch, and (when names is non-null) names[i-1] is that kernel's name, a
 * static string.  events holds max_events events the caller created
 * (hipEventCreate, timing enabled); launches past max_events - 1 are not
 * marked.  *n_events receives the number of events recorded (0 when the
 * problem is rejected).  Results and errors otherwise as msa_forward_v.  The
 * marks add one event record per launch and change nothing else.
 */
msa_status msa_forward_marked(const msa_problem* p, const msa_varlen* vl, const void* q, const void* k, const void* v,
                              const void* index_q, const void* index_k, void* out, int32_t* block_idx, float* lse,
                              void* workspace, size_t workspace_bytes, hipStream_t stream, hipEvent_t* events,
                              int max_events, const char** names, int* n_events);

/* Static description of a status code. */
const char* msa_status_string(msa_status s);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H_ */
