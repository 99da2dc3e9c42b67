"""GPU parity of the KL alignment pass (msa_index_kl) against the fp64 oracle.

Each case runs the forward pass on the GPU (block_idx and lse), then the KL
pass through the C ABI, and compares every checked row with oracle.kl on the
GPU's own block selection.  Tolerance: the GPU's teacher uses the forward's
fp32 lse and fp32 scores of exact bf16 products; their errors (about 1e-6 in
the exponent on these inputs) move each teacher weight by that relative
amount, and the KL by at most that times (1 + entropy + sum_j t_j |z_j|),
under 1e-4 here; the student's fp32 index scores add at most twice their own
error.  The bound below, 1e-3 absolute plus 1e-4 relative, leaves an order of
magnitude of room for the fp32 sums over up to 2048 tokens.
"""
import numpy as np
import pytest

import block_sparse_long_qk_amd as msa
import oracle
import synth
from gpu_helpers import problem, run_gpu, sample_rows, say

pytestmark = pytest.mark.gpu

KL_ABS, KL_REL = 1e-3, 1e-4

CASES = [
    synth.Workload("kl_g8", 1, 2048, 2048, 16, 2, topk=8, seed=2401),
    synth.Workload("kl_g4_ragged_dimx64", 2, 1000, 1000, 8, 2, index_dim=64, topk=4, seed=2402),
    synth.Workload("kl_g16_chunk", 1, 300, 1000, 32, 2, topk=4, q_offset=700, seed=2403),
    synth.Workload("kl_g32", 1, 1536, 1536, 32, 1, topk=5, seed=2404),
    synth.Workload("kl_decode", 3, 1, 5000, 16, 2, topk=8, seed=2405),
    synth.WORKLOADS["prefill_4k"],
]


def run_kl(w, res):
    import torch
    p = problem(w)
    x = res["inputs"]
    kl = torch.full((w.batch, w.h_kv, w.n_q), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(msa.workspace_size(p, msa.OP_INDEX_KL), 256), dtype=torch.uint8, device="cuda")
    msa.index_kl(p, x["q"], x["k"], x["iq"], x["ik"], res["block_idx"], res["lse"], kl, ws)
    torch.cuda.synchronize()
    return kl


def check_kl_rows(w, res, kl, b, g, rows):
    x = oracle.inputs_for_rows(w, b, g, rows)
    sel = res["block_idx"][b, g].cpu().numpy()[rows]
    K, _ = oracle.kv_for_blocks(w, b, g, sel)
    ref = oracle.kl(x["q"], x["pos"], sel, K, x["iq"], x["ik"], w.block_size, w.scale)
    got = kl[b, g].cpu().numpy()[rows].astype(np.float64)
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got)), "non-finite KL"
    assert np.all(err <= KL_ABS + KL_REL * np.abs(ref)), f"max |d| {err.max():.3e} at row {rows[np.argmax(err)]}"
    assert np.all(got > -1e-5), "KL below zero"
    return err.max(), float(np.mean(ref))


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_kl_matches_oracle(w):
    say(f"[gpu] kl {w.name}: B={w.batch} n_q={w.n_q} n_kv={w.n_kv} h={w.h_q}/{w.h_kv} d_idx={w.index_dim} k={w.topk}")
    res = run_gpu(w, with_forward=False)
    kl = run_kl(w, res)
    rows = np.arange(w.n_q) if w.n_q <= 2048 else sample_rows(w, 256, seed=w.seed, whole_blocks=2)
    worst, mean = 0.0, []
    for b in range(w.batch):
        for g in range(w.h_kv):
            e, m = check_kl_rows(w, res, kl, b, g, rows)
            worst = max(worst, e)
            mean.append(m)
    say(f"    KL max |d| = {worst:.3e}, mean KL = {np.mean(mean):.4f}")


@pytest.mark.parametrize("name,n_rand", [("prefill_32k", 48), ("prefill_128k", 16)])
def test_kl_full_size_sampled(name, n_rand):
    import torch
    w = synth.WORKLOADS[name]
    res = run_gpu(w, with_forward=False)
    kl = run_kl(w, res)
    rows = sample_rows(w, n_rand, seed=w.seed, whole_blocks=0)
    worst = 0.0
    for g in range(w.h_kv):
        e, _ = check_kl_rows(w, res, kl, 0, g, rows)
        worst = max(worst, e)
    say(f"    KL max |d| = {worst:.3e}")
    assert bool(torch.isfinite(kl).all())
    del res, kl
    torch.cuda.empty_cache()
