"""GPU parity of the FP8 (OCP E4M3) index branch against the fp64 oracle.

The index inputs are the workloads' bf16 index_q / index_k rounded to E4M3
(nearest even); the oracle scores the same E4M3 values exactly (pool_f8) and
the rules are those of the bf16 tests: pooled scores within the fp32
summation bound (E4M3 products are exact in fp32), the selection bit-exact
outside the 1e-3 gap and epsilon-valid inside it, the attention within the
output tolerances on the selected blocks.  Covers the prefill scoring kernel
(pooled and fused top-k), the decode kernel, index dims 64 and 128, ragged
caches, a chunk at an offset and the full-size workloads on sampled rows.
"""
import numpy as np
import pytest

import synth
from gpu_helpers import (Stats, check_forward_matches_stages, check_groups, check_rows, check_topk_all_rows,
                         run_gpu, sample_rows, say)

pytestmark = pytest.mark.gpu


def fp8(w: synth.Workload, name: str | None = None) -> synth.Workload:
    return w.replace(name=name or ("fp8_" + w.name), index_dtype="fp8")


def _release():
    import torch
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


SMALL = [
    fp8(synth.WORKLOADS["prefill_4k"]),  # index dim 64, planted keys
    synth.Workload("fp8_ragged", 2, 1000, 1000, 8, 2, index_dim=64, topk=4, seed=2301, index_dtype="fp8"),
    synth.Workload("fp8_chunk", 1, 300, 1000, 8, 2, topk=4, q_offset=700, seed=2302, index_dtype="fp8"),
    synth.Workload("fp8_g16_k16", 1, 3000, 3000, 32, 2, topk=16, seed=2303, index_dtype="fp8"),
    # one launch over all key blocks: the fused scoring + top-k path of msa_forward
    synth.Workload("fp8_fused_k8", 1, 8192, 8192, 128, 16, topk=8, seed=2304, index_dtype="fp8"),
    # decode-shaped: the streaming index kernel, index dims 128 and 64
    synth.Workload("fp8_decode", 3, 1, 5000, 16, 2, topk=8, seed=2305, index_dtype="fp8"),
    synth.Workload("fp8_decode_dimx64", 2, 1, 3000, 8, 2, index_dim=64, topk=6, seed=2306, index_dtype="fp8"),
    synth.Workload("fp8_rows_nq4", 2, 4, 3000, 16, 2, topk=6, seed=2307, index_dtype="fp8"),
    synth.Workload("fp8_one_token", 2, 1, 1, 8, 1, seed=2308, index_dtype="fp8"),
]


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_fp8_small(w):
    res = run_gpu(w)
    check_forward_matches_stages(res)
    st = Stats()
    rows = np.arange(w.n_q) if w.n_q <= 3000 else sample_rows(w, 256, seed=w.seed, whole_blocks=3)
    for b in range(w.batch):
        for g in range(w.h_kv):
            check_rows(w, res, b, g, rows, st)
    st.check()
    del res
    _release()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,n_rand,seqs", [("prefill_32k", 48, None), ("prefill_128k", 256, None),
                                               ("decode_256k", 0, (0, 37, 63)), ("chunked_1m", 6, None)])
def test_fp8_full_size_sampled(name, n_rand, seqs):
    """The full-size workloads with E4M3 index inputs: msa_forward (the fused
    scoring + top-k launch at 32K and 128K) equals the three calls bit for bit,
    every 128K row's top-k equals the oracle's on the GPU's fp32 scores, and
    sampled rows match the oracle."""
    w = fp8(synth.WORKLOADS[name])
    res = run_gpu(w, with_forward=True)
    check_forward_matches_stages(res)
    if name == "prefill_128k":
        say(f"    top-k: {check_topk_all_rows(w, res)} rows bit-exact on the GPU's fp32 scores")
    st = Stats()
    plant = synth.plant_spec(w)
    if seqs is None:
        rows = sample_rows(w, n_rand, seed=w.seed, whole_blocks=2 if name == "prefill_128k" else 0)
        check_groups(w, res, 0, rows, st, plant)
    else:
        for b in seqs:
            check_groups(w, res, b, [0], st, plant)
    st.check()
    del res
    _release()


def test_fp8_device_inputs_match_host():
    """The device E4M3 index inputs equal the host ones the oracle reads."""
    import torch
    w = fp8(synth.WORKLOADS["prefill_32k"])  # planted: the planted rows are converted too
    x = synth.device_inputs(w)
    assert x["iq"].dtype == torch.uint8 and x["ik"].dtype == torch.uint8
    rows = np.array([0, 1, 777, 20000, w.n_q - 1])
    host_iq = synth.to_e4m3(synth.host_iq_rows(w, 0, rows))
    dev_iq = x["iq"][0].index_select(0, torch.from_numpy(rows).cuda()).cpu().numpy()
    assert np.array_equal(host_iq, dev_iq)
    plant = synth.plant_spec(w)
    for t in [0, plant.blocks[0][0], w.n_blk - 1]:
        j0, j1 = t * w.block_size, (t + 1) * w.block_size
        assert np.array_equal(synth.to_e4m3(synth.host_ik(w, 0, j0, j1, plant)), x["ik"][0, j0:j1].cpu().numpy())
    say("    E4M3 inputs: device equals host")


@pytest.mark.parametrize("n_q", [4096, 1], ids=["prefill-kernel", "decode-kernel"])
def test_e4m3_run_truncation_model(n_q):
    """Pins the accumulation model the E4M3 pooled tolerance rests on, through
    the C ABI: a product 2^-g of the largest one (2^8) in the same run of 8
    index dims is dropped for g >= 14 (truncated toward zero) and kept for
    g <= 13; in another run it is always kept (fp32 accumulation)."""
    import torch
    import block_sparse_long_qk_amd as msa
    n_kv, d_idx, bk = 4096, 128, 128
    e4m3 = lambda v: torch.tensor(v, dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8)
    iq = torch.zeros((n_q, 1, d_idx), dtype=torch.uint8)
    iq[:, 0, 0] = e4m3(16.0)
    iq[:, 0, 1] = e4m3(1.0)
    iq[:, 0, 8] = e4m3(1.0)
    ik = torch.zeros((n_kv, d_idx), dtype=torch.uint8)
    expect = {}
    t = 0
    for sign in (1.0, -1.0):
        for dim in (1, 8):                 # same run as the large product, or the next run
            for g in range(10, 18):
                j = t * bk                 # the block's first key carries the pattern, the rest score 0
                ik[j, 0] = e4m3(16.0)
                ik[j, dim] = e4m3(sign * 2.0 ** (8 - g))
                small = sign * 2.0 ** (8 - g)
                expect[t] = 256.0 if (dim == 1 and g >= 14) else 256.0 + small
                t += 1
    assert t == n_kv // bk
    p = msa.Problem.make(1, n_q, n_kv, 1, 1, 128, d_idx, bk, 16, index_dtype=msa.DTYPE_FP8_E4M3)
    pooled = torch.full((1, 1, n_q, n_kv // bk), -1.0, dtype=torch.float32, device="cuda")
    msa.index_scores(p, iq.cuda(), ik.cuda(), pooled)
    torch.cuda.synchronize()
    got = pooled[0, 0, -1].cpu().numpy().astype(np.float64)   # the last query sees every block
    want = np.array([expect[u] for u in range(t)])
    say(f"    run-truncation pattern ({'prefill' if n_q > 1 else 'decode'} kernel): "
        f"{int(np.sum(got == want))}/{t} blocks as modelled")
    assert np.array_equal(got, want), np.stack([got, want])
