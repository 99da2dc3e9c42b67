"""A long prefill run in passes over query chunks (msa_problem.chunk_rows)
writes the same bits as one pass: msa_forward and msa_sparse_attn_fwd with
passes of 8192 rows against the same calls in one pass, on the 32K workload,
a two-sequence batch with a ragged last pass, a chunk at an offset, FP8 inputs
and a call without lse.  The single pass is checked against the oracle by the
parity tests; bitwise equality carries that over to the passes."""
import numpy as np
import pytest

import block_sparse_long_qk_amd as msa
import synth
from gpu_helpers import Stats, check_rows, problem, say

pytestmark = pytest.mark.gpu

CASES = [
    (synth.WORKLOADS["prefill_32k"], True),
    (synth.Workload("passes_b2_ragged", 2, 20000, 20000, 16, 2, topk=16, seed=3401), True),
    (synth.Workload("passes_offset", 1, 17000, 20000, 16, 2, topk=8, q_offset=3000, seed=3402), False),
    (synth.Workload("passes_fp8", 1, 16384, 16384, 16, 2, topk=16, seed=3403, index_dtype="fp8", kv_dtype="fp8"),
     True),
]


def _with_chunk(p, c):
    q = msa.Problem.make(p.batch, p.n_q, p.n_kv, p.h_q, p.h_kv, p.head_dim, p.index_dim, p.block_size, p.topk,
                         p.q_offset, p.softmax_scale, p.index_dtype, p.kv_dtype, chunk_rows=c)
    return q


@pytest.mark.parametrize("w,with_lse", CASES, ids=[c[0].name for c in CASES])
def test_passes_equal_one_pass(w, with_lse):
    import torch
    x = synth.device_inputs(w)
    p1 = problem(w)
    pc = _with_chunk(p1, 8192)
    ws1, wsc = msa.workspace_size(p1, msa.OP_FORWARD), msa.workspace_size(pc, msa.OP_FORWARD)
    say(f"[gpu] {w.name}: workspace one pass {ws1 / 2**20:.0f} MiB, passes of 8192 rows {wsc / 2**20:.0f} MiB")
    assert wsc < ws1
    outs = []
    for p in (p1, pc):
        f = msa.alloc_outputs(p, x["q"].device, lse=with_lse)
        f["block_idx"].fill_(-7)
        msa.forward(p, x["q"], x["k"], x["v"], x["iq"], x["ik"], f["out"], f["block_idx"], f["lse"],
                    f["workspace"])
        torch.cuda.synchronize()
        outs.append(f)
    a, c = outs
    assert torch.equal(a["block_idx"], c["block_idx"])
    assert torch.equal(a["out"].view(torch.int16), c["out"].view(torch.int16))
    if with_lse:
        assert torch.equal(a["lse"], c["lse"])
    # msa_sparse_attn_fwd in passes on the same selection
    ws = torch.empty(msa.workspace_size(pc, msa.OP_SPARSE_ATTN), dtype=torch.uint8, device=x["q"].device)
    out2 = torch.empty_like(a["out"])
    lse2 = torch.empty_like(a["lse"]) if with_lse else None
    msa.sparse_attn_fwd(pc, x["q"], x["k"], x["v"], a["block_idx"], out2, lse2, ws)
    torch.cuda.synchronize()
    assert torch.equal(a["out"].view(torch.int16), out2.view(torch.int16))
    if with_lse:
        assert torch.equal(a["lse"], lse2)
    # and a few rows of the chunked call against the oracle, one per pass boundary
    st = Stats()
    res = {"pooled": None, "block_idx": c["block_idx"], "out": c["out"], "lse": c["lse"] if with_lse else lse2}
    if with_lse:
        rows = np.array(sorted({0, 8191, 8192, 16383, 16384, w.n_q - 1} & set(range(w.n_q))))
        pooled = torch.empty((w.batch, w.h_kv, w.n_q, w.n_blk), dtype=torch.float32, device=x["q"].device)
        msa.index_scores(p1, x["iq"], x["ik"], pooled)
        torch.cuda.synchronize()
        res["pooled"] = pooled
        for b in range(w.batch):
            for g in range(w.h_kv):
                check_rows(w, res, b, g, rows, st)
        st.check()
