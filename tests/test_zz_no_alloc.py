"""msa_forward_noalloc (the workspace is the library's fixed device scratch)
against msa_forward with a caller's workspace: bit for bit equal outputs on
two calls in a row, the second smaller than the first (the scratch keeps the
first call's contents), then the first shape again."""
import pytest

import block_sparse_long_qk_amd as msa
import synth
from gpu_helpers import problem, say

pytestmark = pytest.mark.gpu

CALLS = [
    synth.WORKLOADS["prefill_4k"],                                          # 70 MiB of workspace
    synth.Workload("noalloc_decode", 4, 1, 5000, 16, 2, topk=8, seed=3501),  # a few MiB
    synth.Workload("noalloc_prefill_small", 1, 1500, 2000, 16, 2, topk=6, seed=3502),
]


def _run(w, noalloc):
    import torch
    x = synth.device_inputs(w)
    p = problem(w)
    f = msa.alloc_outputs(p, x["q"].device)
    f["out"].fill_(7)
    f["block_idx"].fill_(-7)
    f["lse"].fill_(7)
    if noalloc:
        msa.forward_noalloc(p, x["q"], x["k"], x["v"], x["iq"], x["ik"], f["out"], f["block_idx"], f["lse"])
    else:
        msa.forward(p, x["q"], x["k"], x["v"], x["iq"], x["ik"], f["out"], f["block_idx"], f["lse"], f["workspace"])
    torch.cuda.synchronize()
    return f


def test_noalloc_equals_forward_on_consecutive_calls():
    import torch
    for w in CALLS + CALLS[:1]:
        ws = msa.workspace_size(problem(w), msa.OP_FORWARD)
        say(f"[gpu] noalloc {w.name}: workspace {ws / 2**20:.1f} MiB of {msa.NOALLOC_SCRATCH_BYTES >> 20} MiB")
        a, b = _run(w, False), _run(w, True)
        assert torch.equal(a["block_idx"], b["block_idx"])
        assert torch.equal(a["out"].view(torch.int16), b["out"].view(torch.int16))
        assert torch.equal(a["lse"], b["lse"])
