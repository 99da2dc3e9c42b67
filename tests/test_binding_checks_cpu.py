"""The Python binding checks every tensor before the C call: element type,
contiguity, size against the problem, and that all of them sit on one GPU.
Run on the CPU: host tensors of the right shape reach the device check (the
last one), tensors of a wrong shape, dtype or layout fail earlier, and no call
reaches the library."""
import pytest
import torch

import block_sparse_long_qk_amd as msa


def prob(**kw):
    base = dict(batch=1, n_q=256, n_kv=256, h_q=4, h_kv=1, head_dim=128, index_dim=64, block_size=128, topk=2)
    base.update(kw)
    return msa.Problem.make(**base)


def inputs(p, **over):
    x = {
        "q": torch.zeros((p.batch, p.n_q, p.h_q, p.head_dim), dtype=torch.bfloat16),
        "k": torch.zeros((p.batch, p.h_kv, p.n_kv, p.head_dim), dtype=torch.bfloat16),
        "v": torch.zeros((p.batch, p.h_kv, p.n_kv, p.head_dim), dtype=torch.bfloat16),
        "iq": torch.zeros((p.batch, p.n_q, p.h_kv, p.index_dim), dtype=torch.bfloat16),
        "ik": torch.zeros((p.batch, p.n_kv, p.index_dim), dtype=torch.bfloat16),
        "pooled": torch.zeros((p.batch, p.h_kv, p.n_q, p.n_blk), dtype=torch.float32),
        "bidx": torch.zeros((p.batch, p.h_kv, p.n_q, p.topk), dtype=torch.int32),
        "out": torch.zeros((p.batch, p.n_q, p.h_q, p.head_dim), dtype=torch.bfloat16),
        "lse": torch.zeros((p.batch, p.h_q, p.n_q), dtype=torch.float32),
        "ws": torch.zeros(1 << 12, dtype=torch.uint8),
    }
    x.update(over)
    return x


def call_forward(p, x):
    msa.forward(p, x["q"], x["k"], x["v"], x["iq"], x["ik"], x["out"], x["bidx"], x["lse"], x["ws"], stream=0)


def test_host_tensors_rejected_at_the_device_check():
    p = prob()
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        call_forward(p, inputs(p))
    x = inputs(p)
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        msa.index_scores(p, x["iq"], x["ik"], x["pooled"], stream=0)
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        msa.block_topk(p, x["pooled"], x["bidx"], stream=0)
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        msa.sparse_attn_fwd(p, x["q"], x["k"], x["v"], x["bidx"], x["out"], x["lse"], x["ws"], stream=0)
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        msa.dense_attn_fwd(p, x["q"], x["k"], x["v"], x["out"], x["lse"], stream=0)


@pytest.mark.parametrize("name,bad,match", [
    ("q", torch.zeros((1, 255, 4, 128), dtype=torch.bfloat16), "q holds"),             # one row short
    ("k", torch.zeros((1, 1, 256, 128), dtype=torch.float16), "k has dtype"),           # fp16 is not a K dtype
    ("iq", torch.zeros((1, 256, 1, 64), dtype=torch.uint8), "index_q has dtype"),       # FP8 codes for a bf16 problem
    ("ik", torch.zeros((1, 128, 64), dtype=torch.bfloat16), "index_k holds"),           # half the keys
    ("bidx", torch.zeros((1, 1, 256, 2), dtype=torch.int64), "block_idx has dtype"),
    ("out", torch.zeros((1, 256, 4, 256), dtype=torch.bfloat16)[..., ::2], "out must be contiguous"),
    ("lse", torch.zeros((1, 4, 255), dtype=torch.float32), "lse holds"),
    ("v", None, "v is required"),
    ("q", [0] * 10, "must be a torch tensor"),
])
def test_bad_tensors_rejected(name, bad, match):
    p = prob()
    with pytest.raises(ValueError, match=match):
        call_forward(p, inputs(p, **{name: bad}))


def test_workspace_bytes_beyond_the_tensor_rejected():
    p = prob()
    x = inputs(p)
    with pytest.raises(ValueError, match="exceeds the workspace tensor"):
        msa.forward(p, x["q"], x["k"], x["v"], x["iq"], x["ik"], x["out"], x["bidx"], x["lse"], x["ws"],
                    workspace_bytes=1 << 20, stream=0)


def test_pooled_size_follows_the_block_count():
    p = prob(n_q=256, n_kv=300)   # 3 blocks
    x = inputs(p, pooled=torch.zeros((1, 1, 256, 2), dtype=torch.float32))
    with pytest.raises(ValueError, match="pooled holds"):
        msa.index_scores(p, x["iq"], x["ik"], x["pooled"], stream=0)


def test_fp8_problems_take_codes():
    p = prob(index_dtype=msa.DTYPE_FP8_E4M3, kv_dtype=msa.DTYPE_FP8_E4M3)
    x = inputs(p)
    with pytest.raises(ValueError, match="k has dtype bfloat16"):
        call_forward(p, x)
    x["k"] = torch.zeros((1, 1, 256, 128), dtype=torch.uint8)
    x["v"] = torch.zeros((1, 1, 256, 128), dtype=torch.float8_e4m3fn)
    with pytest.raises(ValueError, match="index_q has dtype bfloat16"):
        call_forward(p, x)
    x["iq"] = torch.zeros((1, 256, 1, 64), dtype=torch.uint8)
    x["ik"] = torch.zeros((1, 256, 64), dtype=torch.uint8)
    with pytest.raises(ValueError, match="must be a GPU tensor"):   # every other check passed
        call_forward(p, x)


def test_varlen_sizes():
    """Packed rows are sized by total_q and paged caches by the pool."""
    p = prob(batch=2, n_q=256, n_kv=256)
    i32 = lambda *s: torch.zeros(s, dtype=torch.int32)
    vl = msa.Varlen.make(qo_lens=i32(2), kv_lens=i32(2), q_starts=i32(2), total_q=300,
                         page_table=i32(2, 2), num_pages=5)
    x = inputs(p, q=torch.zeros((300, 4, 128), dtype=torch.bfloat16),
               out=torch.zeros((300, 4, 128), dtype=torch.bfloat16),
               iq=torch.zeros((300, 1, 64), dtype=torch.bfloat16),
               k=torch.zeros((5, 1, 128, 128), dtype=torch.bfloat16),
               v=torch.zeros((5, 1, 128, 128), dtype=torch.bfloat16),
               ik=torch.zeros((5, 128, 64), dtype=torch.bfloat16))
    args = lambda x: (p, x["q"], x["k"], x["v"], x["iq"], x["ik"], x["out"], x["bidx"], x["lse"], x["ws"])
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        msa.forward(*args(x), stream=0, varlen=vl)
    x["k"] = torch.zeros((4, 1, 128, 128), dtype=torch.bfloat16)   # one page short of the pool
    with pytest.raises(ValueError, match="k holds"):
        msa.forward(*args(x), stream=0, varlen=vl)
    bad = msa.Varlen.make(qo_lens=torch.zeros(2, dtype=torch.int64), q_starts=i32(2), total_q=300)
    x = inputs(p, q=torch.zeros((300, 4, 128), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="qo_lens has dtype"):
        msa.forward(*args(x), stream=0, varlen=bad)


def test_training_calls_checked():
    p = prob(h_q=16, h_kv=2, index_dim=128)
    x = inputs(p)
    kl = torch.zeros((1, 2, 256), dtype=torch.float32)
    with pytest.raises(ValueError, match="kl holds"):
        msa.index_kl(p, x["q"], x["k"], x["iq"], x["ik"], x["bidx"], x["lse"], kl[:, :1], x["ws"], stream=0)
    with pytest.raises(ValueError, match="dout is required"):
        msa.sparse_attn_bwd(p, x["q"], x["k"], x["v"], x["bidx"], x["out"], x["lse"], None, x["q"], x["k"], x["v"],
                            x["ws"], stream=0)
    with pytest.raises(ValueError, match="lse_index is required"):
        msa.index_kl_bwd(p, x["q"], x["k"], x["iq"], x["ik"], x["bidx"], x["lse"], None, x["iq"], x["ik"],
                         workspace=x["ws"], stream=0)


def test_stored_teacher_calls_checked():
    """The teacher-keeping KL pass and the backward that reads the teacher:
    the teacher must be fp16 of teacher_shape(p), lse_index is required, and
    host tensors of the right shapes get as far as the device check."""
    p = prob(h_q=16, h_kv=2, index_dim=128)
    x = inputs(p)
    kl = torch.zeros((1, 2, 256), dtype=torch.float32)
    lz = torch.zeros_like(kl)
    assert msa.teacher_shape(p) == (1, 2, 256, 3, 128)
    teacher = torch.zeros(msa.teacher_shape(p), dtype=torch.float16)
    call = lambda t, l: msa.index_kl_teacher(p, x["q"], x["k"], x["iq"], x["ik"], x["bidx"], x["lse"], kl, l, t,
                                             x["ws"], stream=0)
    with pytest.raises(ValueError, match="teacher has dtype"):
        call(teacher.to(torch.bfloat16), lz)
    with pytest.raises(ValueError, match="teacher holds"):
        call(teacher.reshape(-1)[:1000], lz)
    with pytest.raises(ValueError, match="lse_index is required"):
        call(teacher, None)
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        call(teacher, lz)
    bcall = lambda t, l: msa.index_kl_bwd_teacher(p, x["iq"], x["ik"], x["bidx"], t, l, x["iq"], x["ik"],
                                                  workspace=x["ws"], stream=0)
    with pytest.raises(ValueError, match="teacher has dtype"):
        bcall(teacher.float(), lz)
    with pytest.raises(ValueError, match="lse_index is required"):
        bcall(teacher, None)
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        bcall(teacher, lz)
