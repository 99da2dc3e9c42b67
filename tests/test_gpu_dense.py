"""GPU parity of dense mode (the indexer warmup: both branches over every
visible token) against the fp64 oracle.

msa_dense_attn_fwd is compared with oracle.dense_gqa (itself pinned to
torch's scaled_dot_product_attention on the CPU) under the attention's output
tolerances, on seven shapes and on sampled rows of the benchmarked 128K call;
msa_dense_index_kl, fed the dense lse, with oracle.kl over all visible blocks
under the KL tolerance of the sparse pass (four shapes, and sampled rows of
the benchmarked 128K call).  Two consistency checks tie dense and sparse mode
together: with k * Bk >= n_kv the sparse calls select every block, so they
must agree with the dense ones.
"""
import numpy as np
import pytest

import block_sparse_long_qk_amd as msa
import oracle
import synth
from gpu_helpers import LSE_ABS, OUT_MAX_ABS, OUT_MEAN_ABS, Stats, problem, run_gpu, sample_rows, say
from test_gpu_kl import KL_ABS, KL_REL

pytestmark = pytest.mark.gpu

ATTN_CASES = [
    synth.Workload("dense_ragged", 1, 1000, 1000, 8, 2, seed=2501),
    synth.Workload("dense_chunk_b2", 2, 300, 1000, 8, 2, q_offset=700, seed=2502),
    synth.Workload("dense_g1", 1, 777, 777, 4, 4, seed=2503),
    synth.Workload("dense_g16", 1, 1536, 1536, 32, 2, seed=2504),
    synth.Workload("dense_g128", 1, 512, 512, 128, 1, seed=2505),
    synth.Workload("dense_decode", 3, 1, 5000, 16, 2, seed=2506),
    synth.Workload("dense_8k", 1, 8192, 8192, 16, 2, seed=2507),
]

KL_CASES = [
    synth.Workload("dkl_g8", 1, 2048, 2048, 16, 2, seed=2511),
    synth.Workload("dkl_g4_dimx64", 2, 700, 700, 8, 2, index_dim=64, seed=2512),
    synth.Workload("dkl_g16_chunk", 1, 300, 1000, 32, 2, q_offset=700, seed=2513),
    synth.Workload("dkl_g32", 1, 1024, 1024, 32, 1, seed=2514),
]


def dense_gpu(w, x=None):
    import torch
    x = synth.device_inputs(w) if x is None else x
    p = problem(w)
    out = torch.empty((w.batch, w.n_q, w.h_q, w.head_dim), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.batch, w.h_q, w.n_q), dtype=torch.float32, device="cuda")
    msa.dense_attn_fwd(p, x["q"], x["k"], x["v"], out, lse)
    torch.cuda.synchronize()
    return x, out, lse


@pytest.mark.parametrize("w", ATTN_CASES, ids=[w.name for w in ATTN_CASES])
def test_dense_attention_matches_oracle(w):
    import torch
    say(f"[gpu] dense attention {w.name}: B={w.batch} n_q={w.n_q} n_kv={w.n_kv} h={w.h_q}/{w.h_kv}")
    x, out, lse = dense_gpu(w)
    rows = np.arange(w.n_q) if w.n_q <= 2048 else sample_rows(w, 128, seed=w.seed, whole_blocks=2)
    st = Stats()
    idx = torch.from_numpy(rows).cuda()
    for b in range(w.batch):
        for g in range(w.h_kv):
            G = w.group
            q_rows = synth.host_q_rows(w, b, rows)[:, g * G:(g + 1) * G, :]
            K = synth.host_kv(w, "k", b, g, 0, w.n_kv)
            V = synth.host_kv(w, "v", b, g, 0, w.n_kv)
            ref_o, ref_l = oracle.dense_gqa(q_rows, w.offset + rows, K, V, w.scale)
            st.add_out(out[b].index_select(0, idx)[:, g * G:(g + 1) * G].float().cpu().numpy(), ref_o)
            st.add_lse(lse[b, g * G:(g + 1) * G].index_select(1, idx).cpu().numpy().T, ref_l)
    st.check()


def test_dense_attention_128k_sampled():
    """The benchmarked 128K dense call on sampled rows, all groups and heads:
    the first and last positions (one key and every key visible), both sides of
    the first block edge, and random positions."""
    import torch
    w = synth.WORKLOADS["prefill_128k"]
    say(f"[gpu] dense attention {w.name}: sampled rows")
    x, out, lse = dense_gpu(w)
    rng = np.random.default_rng(w.seed)
    rows = np.unique(np.concatenate([[0, 127, 128, w.n_q - 1], rng.integers(0, w.n_q, 3)])).astype(np.int64)
    st = Stats()
    idx = torch.from_numpy(rows).cuda()
    G = w.group
    for g in range(w.h_kv):
        q_rows = synth.host_q_rows(w, 0, rows)[:, g * G:(g + 1) * G, :]
        n_seen = int(w.offset + rows.max()) + 1
        K = synth.host_kv(w, "k", 0, g, 0, n_seen)
        V = synth.host_kv(w, "v", 0, g, 0, n_seen)
        ref_o, ref_l = oracle.dense_gqa(q_rows, w.offset + rows, K, V, w.scale)
        st.add_out(out[0].index_select(0, idx)[:, g * G:(g + 1) * G].float().cpu().numpy(), ref_o)
        st.add_lse(lse[0, g * G:(g + 1) * G].index_select(1, idx).cpu().numpy().T, ref_l)
    st.check()


@pytest.mark.parametrize("w", KL_CASES, ids=[w.name for w in KL_CASES])
def test_dense_kl_matches_oracle(w):
    import torch
    say(f"[gpu] dense KL {w.name}")
    x, out, lse = dense_gpu(w)
    p = problem(w)
    kl = torch.full((w.batch, w.h_kv, w.n_q), float("nan"), dtype=torch.float32, device="cuda")
    msa.dense_index_kl(p, x["q"], x["k"], x["iq"], x["ik"], lse, kl)
    torch.cuda.synchronize()
    rows = np.arange(w.n_q)
    worst = 0.0
    for b in range(w.batch):
        for g in range(w.h_kv):
            xr = oracle.inputs_for_rows(w, b, g, rows)
            local = xr["pos"] // w.block_size
            sel = np.full((len(rows), w.n_blk), -1, np.int32)
            for r, l in enumerate(local):
                sel[r, :l + 1] = np.arange(l + 1)
            K = synth.host_kv(w, "k", b, g, 0, w.n_kv)
            ref = oracle.kl(xr["q"], xr["pos"], sel, K, xr["iq"], xr["ik"], w.block_size, w.scale)
            got = kl[b, g].cpu().numpy().astype(np.float64)
            err = np.abs(got - ref)
            assert np.all(np.isfinite(got))
            assert np.all(err <= KL_ABS + KL_REL * np.abs(ref)), f"max |d| {err.max():.3e}"
            worst = max(worst, float(err.max()))
    say(f"    dense KL max |d| = {worst:.3e}")


def test_dense_kl_128k_sampled():
    """The benchmarked 128K dense KL (fed the dense lse) on sampled rows of
    every group: the first and last positions, both sides of the first block
    edge, and random positions."""
    import torch
    w = synth.WORKLOADS["prefill_128k"]
    say(f"[gpu] dense KL {w.name}: sampled rows")
    x, out, lse = dense_gpu(w)
    p = problem(w)
    kl = torch.full((w.batch, w.h_kv, w.n_q), float("nan"), dtype=torch.float32, device="cuda")
    msa.dense_index_kl(p, x["q"], x["k"], x["iq"], x["ik"], lse, kl)
    torch.cuda.synchronize()
    rng = np.random.default_rng(w.seed + 1)
    rows = np.unique(np.concatenate([[0, 127, 128, w.n_q - 1], rng.integers(0, w.n_q, 3)])).astype(np.int64)
    worst = 0.0
    for g in range(w.h_kv):
        xr = oracle.inputs_for_rows(w, 0, g, rows)
        local = xr["pos"] // w.block_size
        sel = np.full((len(rows), int(local.max()) + 1), -1, np.int32)
        for r, l in enumerate(local):
            sel[r, :l + 1] = np.arange(l + 1)
        K = synth.host_kv(w, "k", 0, g, 0, int(xr["pos"].max()) + 1)
        ref = oracle.kl(xr["q"], xr["pos"], sel, K, xr["iq"], xr["ik"], w.block_size, w.scale)
        got = kl[0, g].cpu().numpy().astype(np.float64)[rows]
        err = np.abs(got - ref)
        assert np.all(np.isfinite(got))
        assert np.all(err <= KL_ABS + KL_REL * np.abs(ref)), f"max |d| {err.max():.3e}"
        worst = max(worst, float(err.max()))
    say(f"    dense KL max |d| = {worst:.3e}")


def test_sparse_with_every_block_equals_dense():
    """k * Bk >= n_kv: the sparse path attends every visible token, so its
    output, lse and KL agree with dense mode's."""
    import torch
    w = synth.Workload("all_blocks", 1, 2000, 2000, 16, 2, topk=16, seed=2520)
    res = run_gpu(w, with_forward=False)
    x, out, lse = dense_gpu(w, res["inputs"])
    d = (res["out"].float() - out.float()).abs()
    say(f"    sparse vs dense: out max |d| {d.max().item():.3e}, lse max |d| {(res['lse'] - lse).abs().max().item():.3e}")
    assert d.max().item() <= OUT_MAX_ABS and d.mean().item() <= OUT_MEAN_ABS
    assert (res["lse"] - lse).abs().max().item() <= LSE_ABS
    p = problem(w)
    kl_s = torch.empty((1, w.h_kv, w.n_q), dtype=torch.float32, device="cuda")
    kl_d = torch.empty_like(kl_s)
    ws = torch.empty(msa.workspace_size(p, msa.OP_INDEX_KL), dtype=torch.uint8, device="cuda")
    msa.index_kl(p, x["q"], x["k"], x["iq"], x["ik"], res["block_idx"], res["lse"], kl_s, ws)
    msa.dense_index_kl(p, x["q"], x["k"], x["iq"], x["ik"], lse, kl_d)
    torch.cuda.synchronize()
    assert (kl_s - kl_d).abs().max().item() <= KL_ABS
