"""The C ABI without a GPU: the library loads, exports every entry point that
include/msa.h declares, sizes workspaces, and rejects bad arguments on the
host before any HIP call (so these calls never reach the device)."""
import ctypes
import os
import re

import pytest

import block_sparse_long_qk_amd as msa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(msa_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = msa.library()
    names = declared_functions()
    assert set(names) == set(msa.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    assert msa.status_string(msa.OK) == "ok"
    assert "workspace" in msa.status_string(msa.ERR_WORKSPACE_TOO_SMALL)
    assert msa.status_string(99) == "unknown status"


def prob(**kw):
    base = dict(batch=1, n_q=4096, n_kv=4096, h_q=4, h_kv=1, head_dim=128, index_dim=64, block_size=128, topk=16)
    base.update(kw)
    return msa.Problem.make(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(h_q=6, h_kv=4), msa.ERR_INVALID_ARGUMENT),          # H_q % H_kv != 0
    (dict(n_q=10, n_kv=8), msa.ERR_INVALID_ARGUMENT),         # q_offset + n_q > n_kv
    (dict(q_offset=5, n_q=4092), msa.ERR_INVALID_ARGUMENT),
    (dict(q_offset=-2), msa.ERR_INVALID_ARGUMENT),
    (dict(topk=0), msa.ERR_INVALID_ARGUMENT),
    (dict(batch=0), msa.ERR_INVALID_ARGUMENT),
    (dict(softmax_scale=float("inf")), msa.ERR_INVALID_ARGUMENT),
    (dict(head_dim=64), msa.ERR_UNSUPPORTED),
    (dict(index_dim=96), msa.ERR_UNSUPPORTED),
    (dict(block_size=64), msa.ERR_UNSUPPORTED),
    (dict(topk=65), msa.ERR_UNSUPPORTED),
    (dict(h_q=256, h_kv=1), msa.ERR_UNSUPPORTED),             # G > 128
    (dict(batch=64, n_q=262144, n_kv=262144, h_kv=8, h_q=64, topk=64), msa.ERR_INVALID_ARGUMENT),  # int32 overflow
    (dict(index_dtype=2), msa.ERR_INVALID_ARGUMENT),         # unknown index element type
    (dict(index_dtype=-1), msa.ERR_INVALID_ARGUMENT),
    (dict(kv_dtype=2), msa.ERR_INVALID_ARGUMENT),            # unknown K/V element type
    (dict(kv_dtype=-1), msa.ERR_INVALID_ARGUMENT),
])
def test_invalid_problems_rejected(kw, status):
    p = prob(**kw)
    n = ctypes.c_size_t(0)
    assert msa.library().msa_workspace_size(ctypes.byref(p), msa.OP_INDEX_SCORES, ctypes.byref(n)) == status
    # the compute entry points reject it before touching the device
    fake = 1 << 20
    assert msa.library().msa_index_scores(ctypes.byref(p), fake, fake, fake, None) == status
    assert msa.library().msa_block_topk(ctypes.byref(p), fake, fake, None) == status


def test_null_and_misaligned_pointers_rejected():
    p = prob()
    lib = msa.library()
    ok = 1 << 20
    assert lib.msa_index_scores(ctypes.byref(p), None, ok, ok, None) == msa.ERR_INVALID_ARGUMENT
    assert lib.msa_index_scores(ctypes.byref(p), ok + 2, ok, ok, None) == msa.ERR_INVALID_ARGUMENT
    assert lib.msa_block_topk(ctypes.byref(p), ok, ok + 4, None) == msa.ERR_INVALID_ARGUMENT
    assert lib.msa_sparse_attn_fwd(ctypes.byref(p), ok, ok, ok, ok, ok, None, None, 1 << 30,
                                   None) == msa.ERR_INVALID_ARGUMENT
    assert lib.msa_sparse_attn_fwd(ctypes.byref(p), ok, ok, ok, ok, ok, ok + 8, ok, 1 << 30,
                                   None) == msa.ERR_INVALID_ARGUMENT
    assert lib.msa_forward(None, ok, ok, ok, ok, ok, ok, ok, None, ok, 1 << 30, None) == msa.ERR_INVALID_ARGUMENT
    n = ctypes.c_size_t(0)
    assert lib.msa_workspace_size(ctypes.byref(p), 7, ctypes.byref(n)) == msa.ERR_INVALID_ARGUMENT
    assert lib.msa_workspace_size(ctypes.byref(p), 0, None) == msa.ERR_INVALID_ARGUMENT


def test_workspace_too_small_rejected():
    p = prob()
    need = msa.workspace_size(p, msa.OP_FORWARD)
    ok = 1 << 20
    lib = msa.library()
    assert lib.msa_forward(ctypes.byref(p), ok, ok, ok, ok, ok, ok, ok, None, ok, need - 1,
                           None) == msa.ERR_WORKSPACE_TOO_SMALL
    need_a = msa.workspace_size(p, msa.OP_SPARSE_ATTN)
    assert lib.msa_sparse_attn_fwd(ctypes.byref(p), ok, ok, ok, ok, ok, None, ok, need_a - 1,
                                   None) == msa.ERR_WORKSPACE_TOO_SMALL


def test_workspace_sizes():
    p = prob()
    assert msa.workspace_size(p, msa.OP_INDEX_SCORES) == 0
    assert msa.workspace_size(p, msa.OP_BLOCK_TOPK) == 0
    a = msa.workspace_size(p, msa.OP_SPARSE_ATTN)
    f = msa.workspace_size(p, msa.OP_FORWARD)
    pooled = 4 * p.batch * p.h_kv * p.n_q * p.n_blk
    assert f >= a + pooled
    # partial outputs dominate: one [G, d] slab of 12-bit codes per (row, slot),
    # two exponent bytes per 64 values and a 4-byte log-sum-exp per head
    slots = p.batch * p.h_kv * p.n_q * p.topk * (p.h_q // p.h_kv)
    assert a >= slots * (128 * 12 // 8 + 4 + 4)
    big = msa.Problem.make(1, 131072, 131072, 64, 8)
    # scoring and top-k run as one launch here: no pooled scores in the workspace
    assert msa.workspace_size(big, msa.OP_FORWARD) == msa.workspace_size(big, msa.OP_SPARSE_ATTN)
    assert msa.workspace_size(big, msa.OP_FORWARD) < 40 << 30   # fits one MI355X comfortably


def test_forward_workspace_bounded_at_1m():
    """A 1M-token prefill runs in passes of MSA_DEFAULT_CHUNK_ROWS query rows:
    its workspace is one pass's, under 64 GiB, where one pass over all rows
    would need several hundred GiB."""
    one_m = 1 << 20
    p = msa.Problem.make(1, one_m, one_m, 64, 8)
    f = msa.workspace_size(p, msa.OP_FORWARD)
    a = msa.workspace_size(p, msa.OP_SPARSE_ATTN)
    assert f <= 64 << 30 and a <= 64 << 30
    per_pass_partials = 8 * msa.DEFAULT_CHUNK_ROWS * 17 * 8 * (128 * 12 // 8)  # 12-bit codes
    assert f >= per_pass_partials
    # smaller passes, smaller workspace; a value not on the alignment rounds down
    small = msa.workspace_size(msa.Problem.make(1, one_m, one_m, 64, 8, chunk_rows=16384), msa.OP_FORWARD)
    assert small < f / 4
    assert msa.workspace_size(msa.Problem.make(1, one_m, one_m, 64, 8, chunk_rows=16384 + 5000),
                              msa.OP_FORWARD) == small
    # several sequences: still one pass's workspace
    two = msa.Problem.make(2, 262144, 262144, 64, 8)
    assert msa.workspace_size(two, msa.OP_FORWARD) <= 64 << 30


def test_chunk_rows_at_or_above_n_q_is_one_pass():
    """n_q at or below the pass size: the workspace of a single pass, whatever chunk_rows says."""
    base = msa.workspace_size(msa.Problem.make(1, 32768, 32768, 64, 8), msa.OP_FORWARD)
    for c in (32768, 40000, 1 << 20):
        assert msa.workspace_size(msa.Problem.make(1, 32768, 32768, 64, 8, chunk_rows=c), msa.OP_FORWARD) == base
    # passes of 8192 rows (the minimum): a quarter of the partials, plus pooled scores when
    # 8192 rows cannot run scoring and top-k as one launch
    c8 = msa.workspace_size(msa.Problem.make(1, 32768, 32768, 64, 8, chunk_rows=8192), msa.OP_FORWARD)
    a8 = msa.workspace_size(msa.Problem.make(1, 32768, 32768, 64, 8, chunk_rows=8192), msa.OP_SPARSE_ATTN)
    assert a8 < base / 3 and c8 >= a8


def test_decode_and_chunked_offsets_accepted():
    assert msa.workspace_size(msa.Problem.make(64, 1, 262144, 64, 8), msa.OP_FORWARD) > 0
    assert msa.workspace_size(msa.Problem.make(1, 8192, 1048576, 64, 8, q_offset=1040384), msa.OP_FORWARD) > 0


@pytest.mark.parametrize("p_kw,vl_kw", [
    (dict(q_offset=0), dict(qo_lens=1 << 20)),                       # lengths need bottom-right alignment
    (dict(q_offset=0), dict(kv_lens=1 << 20)),
    (dict(), dict(q_starts=1 << 20, total_q=0)),                       # packed rows need their count
    (dict(), dict(page_table=1 << 20, pages_per_seq=31, num_pages=64)),  # fewer page slots than blocks (32)
    (dict(), dict(page_table=1 << 20, pages_per_seq=32, num_pages=0)),
])
def test_invalid_varlen_rejected(p_kw, vl_kw):
    p = prob(**p_kw)
    vl = msa.Varlen(**vl_kw)
    lib = msa.library()
    fake = 1 << 20
    V = ctypes.byref(vl)
    assert lib.msa_index_scores_v(ctypes.byref(p), V, fake, fake, fake, None) == msa.ERR_INVALID_ARGUMENT
    assert lib.msa_block_topk_v(ctypes.byref(p), V, fake, fake, None) == msa.ERR_INVALID_ARGUMENT
    assert lib.msa_sparse_attn_fwd_v(ctypes.byref(p), V, fake, fake, fake, fake, fake, None, fake, 1 << 40,
                                     None) == msa.ERR_INVALID_ARGUMENT
    assert lib.msa_forward_v(ctypes.byref(p), V, fake, fake, fake, fake, fake, fake, fake, None, fake, 1 << 40,
                             None) == msa.ERR_INVALID_ARGUMENT


def test_null_varlen_is_the_plain_call():
    # same rejection as the plain call for a bad problem, and no crash on NULL
    p = prob(h_q=6, h_kv=4)
    lib = msa.library()
    fake = 1 << 20
    assert lib.msa_block_topk_v(ctypes.byref(p), None, fake, fake, None) == msa.ERR_INVALID_ARGUMENT


def test_problem_struct_layout():
    """The ctypes mirror of msa_problem has the C layout: nine int32, the
    int64 offset on an 8-byte boundary, the float scale, the int32 dtype."""
    P = msa.Problem
    assert P.q_offset.offset == 40 and P.softmax_scale.offset == 48 and P.index_dtype.offset == 52
    assert P.kv_dtype.offset == 56 and P.chunk_rows.offset == 60
    assert ctypes.sizeof(P) == 64


def test_fp8_index_problems_accepted():
    for d_idx in (64, 128):
        p = prob(index_dim=d_idx, index_dtype=msa.DTYPE_FP8_E4M3)
        n = ctypes.c_size_t(0)
        assert msa.library().msa_workspace_size(ctypes.byref(p), msa.OP_FORWARD, ctypes.byref(n)) == msa.OK
        assert n.value == msa.workspace_size(prob(index_dim=d_idx), msa.OP_FORWARD)


@pytest.mark.parametrize("kw", [dict(h_q=4, h_kv=2), dict(h_q=64, h_kv=1), dict(index_dtype=1),
                                dict(h_q=12, h_kv=2)])
def test_index_kl_unsupported_shapes(kw):
    """The KL pass and its backward take G in {4, 8, 16, 32} and bf16 index inputs."""
    p = prob(**kw)
    n = ctypes.c_size_t(0)
    for op in (msa.OP_INDEX_KL, msa.OP_INDEX_KL_BWD):
        assert msa.library().msa_workspace_size(ctypes.byref(p), op, ctypes.byref(n)) == msa.ERR_UNSUPPORTED


def test_index_kl_workspace_is_smaller_than_attention():
    p = prob(h_q=8, h_kv=1)
    assert 0 < msa.workspace_size(p, msa.OP_INDEX_KL) < msa.workspace_size(p, msa.OP_SPARSE_ATTN)


def test_index_kl_bwd_workspace():
    """The plan, one bf16 d_index_q partial per (row, slot) and an fp32 d_index_k
    share per (group, key): at least those two buffers' bytes."""
    B, n_q, n_kv, h_kv, d_idx, k = 1, 4096, 4096, 2, 128, 8
    p = prob(batch=B, n_q=n_q, n_kv=n_kv, h_q=16, h_kv=h_kv, index_dim=d_idx, topk=k)
    need = 2 * B * h_kv * n_q * (k + 1) * d_idx + 4 * B * h_kv * n_kv * d_idx
    assert msa.workspace_size(p, msa.OP_INDEX_KL_BWD) >= need


def test_index_kl_bwd_rejects_null_lse_index():
    """lse_index is required (the student's normaliser); nothing is launched."""
    p = prob(h_q=16, h_kv=2)
    fake = ctypes.c_void_p(4096)
    L = msa.library()
    rc = L.msa_index_kl_bwd(ctypes.byref(p), fake, fake, fake, fake, fake, fake, None, None, fake, fake, fake,
                            1 << 40, None)
    assert rc == msa.ERR_INVALID_ARGUMENT


def test_fp8_kv_forward_accepted_with_the_same_workspace():
    """FP8 K/V changes how the attention stages K and V, not its workspace."""
    for op in (msa.OP_SPARSE_ATTN, msa.OP_FORWARD):
        assert msa.workspace_size(prob(kv_dtype=msa.DTYPE_FP8_E4M3), op) == msa.workspace_size(prob(), op)


@pytest.mark.parametrize("op", ["OP_INDEX_KL", "OP_SPARSE_ATTN_BWD", "OP_INDEX_KL_BWD"])
def test_fp8_kv_training_calls_unsupported(op):
    """The KL pass and both backward passes take bf16 K/V only."""
    p = prob(h_q=16, h_kv=2, kv_dtype=msa.DTYPE_FP8_E4M3)
    n = ctypes.c_size_t(0)
    assert msa.library().msa_workspace_size(ctypes.byref(p), getattr(msa, op), ctypes.byref(n)) == \
        msa.ERR_UNSUPPORTED
    assert msa.workspace_size(prob(h_q=16, h_kv=2), getattr(msa, op)) > 0



def test_noalloc_rejects_problems_beyond_its_scratch():
    """msa_forward_noalloc checks the workspace a problem needs against its
    fixed scratch on the host, before any HIP call."""
    lib = msa.library()
    ok = 1 << 20
    big = msa.Problem.make(1, 32768, 32768, 64, 8)
    assert msa.workspace_size(big, msa.OP_FORWARD) > msa.NOALLOC_SCRATCH_BYTES
    assert lib.msa_forward_noalloc(ctypes.byref(big), ok, ok, ok, ok, ok, ok, ok, None,
                                   None) == msa.ERR_WORKSPACE_TOO_SMALL
    bad = prob(h_q=6, h_kv=4)
    assert lib.msa_forward_noalloc(ctypes.byref(bad), ok, ok, ok, ok, ok, ok, ok, None,
                                   None) == msa.ERR_INVALID_ARGUMENT
    # the 256K decode step and the 4K prefill fit
    assert msa.workspace_size(msa.Problem.make(64, 1, 262144, 64, 8), msa.OP_FORWARD) <= msa.NOALLOC_SCRATCH_BYTES
    assert msa.workspace_size(prob(), msa.OP_FORWARD) <= msa.NOALLOC_SCRATCH_BYTES


def test_header_constants_match_binding():
    """The binding's copies of the header's size constants."""
    import re
    defs = {m[0]: int(m[1]) << int(m[2] or 0)
            for m in re.findall(r"#define (MSA_\w+) \(?(?:\(size_t\))?(\d+)(?: << (\d+))?", open(HEADER).read())}
    assert defs["MSA_DEFAULT_CHUNK_ROWS"] == msa.DEFAULT_CHUNK_ROWS
    assert defs["MSA_CHUNK_ALIGN"] == msa.CHUNK_ALIGN
    assert defs["MSA_NOALLOC_SCRATCH_BYTES"] == msa.NOALLOC_SCRATCH_BYTES
