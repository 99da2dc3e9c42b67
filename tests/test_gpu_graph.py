"""msa_forward under HIP graph capture.

The library enqueues kernels only (no memset, copy, synchronisation or
allocation), so a forward step can be captured once and replayed, as a serving
loop would for decode.  Each replay must reproduce the eager call bit for bit:
the outputs are poisoned by eager kernels between replays (and the workspace
keeps whatever the previous replay left), so every replay has to rebuild its
selection, gather plan and partials itself.
"""
import pytest

import block_sparse_long_qk_amd as msa
import synth
from gpu_helpers import problem, say

pytestmark = pytest.mark.gpu

CASES = [
    synth.Workload("graph_decode", 4, 1, 6000, 16, 2, topk=8, seed=2901),
    synth.Workload("graph_prefill", 1, 2048, 2048, 16, 2, topk=8, seed=2902),
    synth.Workload("graph_prefill_fp8", 2, 700, 1500, 8, 2, topk=4, seed=2903, index_dtype="fp8", kv_dtype="fp8"),
]


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_forward_graph_replays_equal_eager(w):
    import torch
    say(f"[gpu] graph {w.name}: B={w.batch} n_q={w.n_q} n_kv={w.n_kv} h={w.h_q}/{w.h_kv} k={w.topk}")
    p = problem(w)
    x = synth.device_inputs(w)
    f = msa.alloc_outputs(p)

    def step():
        msa.forward(p, x["q"], x["k"], x["v"], x["iq"], x["ik"], f["out"], f["block_idx"], f["lse"], f["workspace"])

    step()
    torch.cuda.synchronize()
    ref = {key: f[key].clone() for key in ("out", "block_idx", "lse")}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # a warm call on the capture stream before capturing
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        f["out"].fill_(float("nan"))
        f["block_idx"].fill_(-77)
        f["lse"].fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(f["block_idx"], ref["block_idx"]), f"replay {rep}: block_idx"
        assert torch.equal(f["out"].view(torch.int16), ref["out"].view(torch.int16)), f"replay {rep}: out"
        assert torch.equal(f["lse"], ref["lse"]), f"replay {rep}: lse"
    del g
