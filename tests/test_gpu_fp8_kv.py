"""GPU parity of the main branch over FP8 (OCP E4M3) K and V caches against
the fp64 oracle.

K and V are the workloads' bf16 caches rounded to E4M3 (nearest even); the
kernels widen every code to bf16 as they stage it, and the oracle attends over
the values the codes represent (oracle.kv_values_bf16: E4M3 decoded by the
pinned oracle_e4m3_decode, exact in bf16).  Everything after the load is the
bf16 path's arithmetic, so the rules are those of the bf16 tests: the
selection (index branch unchanged) bit-exact outside the 1e-3 gap, outputs
within max |d| <= 1e-2 and mean |d| <= 1e-3 on the selected blocks, msa_forward
equal to the separate calls.  Covers the prefill tiles and the local/merge
kernel, the decode (row) kernel for up to 8 and 16 heads per group, a chunk at
an offset, FP8 on both branches and the full-size workloads on sampled rows;
paged FP8 caches are covered by the varlen tests.
"""
import numpy as np
import pytest

import synth
from gpu_helpers import Stats, check_forward_matches_stages, check_rows, run_gpu, sample_rows, say

pytestmark = pytest.mark.gpu


def kv8(w: synth.Workload, name: str | None = None) -> synth.Workload:
    return w.replace(name=name or ("kv8_" + w.name), kv_dtype="fp8")


def _release():
    import torch
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


SMALL = [
    kv8(synth.WORKLOADS["prefill_4k"]),  # index dim 64, planted keys
    synth.Workload("kv8_ragged", 2, 1000, 1000, 8, 2, index_dim=64, topk=4, seed=2801, kv_dtype="fp8"),
    synth.Workload("kv8_chunk", 1, 300, 1000, 8, 2, topk=4, q_offset=700, seed=2802, kv_dtype="fp8"),
    synth.Workload("kv8_g16_k16", 1, 3000, 3000, 32, 2, topk=16, seed=2803, kv_dtype="fp8"),
    synth.Workload("kv8_g1", 1, 777, 777, 4, 4, topk=3, seed=2804, kv_dtype="fp8"),
    # decode-shaped: the row kernel, up to 8 and up to 16 heads per group
    synth.Workload("kv8_decode", 3, 1, 5000, 16, 2, topk=8, seed=2805, kv_dtype="fp8"),
    synth.Workload("kv8_decode_g16", 2, 1, 3000, 32, 2, topk=6, seed=2806, kv_dtype="fp8"),
    synth.Workload("kv8_rows_nq4", 2, 4, 3000, 16, 2, topk=6, seed=2807, kv_dtype="fp8"),
    synth.Workload("kv8_one_token", 2, 1, 1, 8, 1, seed=2808, kv_dtype="fp8"),
    # FP8 on both branches
    synth.Workload("kv8_both", 1, 2048, 2048, 16, 2, topk=8, seed=2809, kv_dtype="fp8", index_dtype="fp8"),
]


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_fp8_kv_small(w):
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


@pytest.mark.parametrize("name,n_rand", [("prefill_32k", 48), ("prefill_128k", 16), ("decode_256k", 0)])
def test_fp8_kv_full_size_sampled(name, n_rand):
    w = kv8(synth.WORKLOADS[name])
    say(f"[gpu] {w.name}: full size, sampled rows")
    res = run_gpu(w, with_forward=False)
    st = Stats()
    if w.n_q == 1:
        for b in range(0, w.batch, 7):
            for g in range(w.h_kv):
                check_rows(w, res, b, g, [0], st)
    else:
        rows = sample_rows(w, n_rand, seed=w.seed, whole_blocks=1)
        for g in range(w.h_kv):
            check_rows(w, res, 0, g, rows, st)
    st.check()
    del res
    _release()
