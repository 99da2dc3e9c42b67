"""msa_block_topk alone on crafted fp32 score tensors: every row must equal the
oracle's selection on the same values, bit for bit (ties, signed zeros, rows
that defeat the kernel's fast threshold, rows of every visible length)."""
import numpy as np
import pytest

import block_sparse_long_qk_amd as msa
import oracle
from gpu_helpers import say

pytestmark = pytest.mark.gpu


def run_topk(pooled_np, n_q, n_kv, h_kv, k, q_offset=-1):
    import torch
    p = msa.Problem.make(1, n_q, n_kv, 8 * h_kv, h_kv, topk=k, q_offset=q_offset)
    pooled = torch.from_numpy(pooled_np.astype(np.float32)).cuda()
    bidx = torch.full((1, h_kv, n_q, k), -7, dtype=torch.int32, device="cuda")
    msa.block_topk(p, pooled, bidx)
    torch.cuda.synchronize()
    return bidx.cpu().numpy()


def check(pooled_np, n_q, n_kv, h_kv, k, q_offset=-1, name=""):
    say(f"[gpu] top-k {name}: n_q={n_q} n_kv={n_kv} h_kv={h_kv} k={k}")
    got = run_topk(pooled_np, n_q, n_kv, h_kv, k, q_offset)
    off = n_kv - n_q if q_offset == -1 else q_offset
    pos = off + np.arange(n_q)
    n_blk = pooled_np.shape[-1]
    vis = np.arange(n_blk)[None, :] <= (pos // 128)[:, None]
    for g in range(h_kv):
        ref = oracle.select(np.where(vis, pooled_np[0, g].astype(np.float64), np.nan), pos, 128, k)
        bad = np.nonzero(np.any(ref != got[0, g], axis=1))[0]
        assert bad.size == 0, f"group {g} rows {bad[:5]}: got {got[0, g, bad[0]]} want {ref[bad[0]]}"


N = 128 * 300


@pytest.mark.parametrize("k", [1, 2, 16, 64])
def test_random_scores(k):
    rng = np.random.default_rng(3000 + k)
    pooled = rng.standard_normal((1, 2, N, N // 128)).astype(np.float32) * 30
    check(pooled, N, N, 2, k, name="random")


def test_heavy_ties():
    rng = np.random.default_rng(3100)
    pooled = rng.integers(-2, 3, size=(1, 2, N, N // 128)).astype(np.float32)
    check(pooled, N, N, 2, 16, name="ties")


def test_signed_zeros():
    rng = np.random.default_rng(3200)
    pooled = np.where(rng.random((1, 1, N, N // 128)) < 0.5, np.float32(-0.0), np.float32(0.0))
    pooled[..., ::7] = -1.0
    check(pooled.astype(np.float32), N, N, 1, 16, name="signed zeros")


def test_all_equal():
    pooled = np.full((1, 1, N, N // 128), 3.25, np.float32)
    check(pooled, N, N, 1, 16, name="all equal")


def test_periodic_rows_take_the_exact_path():
    """Scores that depend only on the lane a block falls in: hundreds of
    blocks pass the lane-maxima threshold, so the exact search runs."""
    t = np.arange(N // 128)
    row = -(t % 64).astype(np.float32)
    pooled = np.broadcast_to(row, (1, 1, N, N // 128)).copy()
    check(pooled, N, N, 1, 16, name="periodic")


def test_long_rows_8192_blocks():
    rng = np.random.default_rng(3300)
    n_kv, n_q = 1 << 20, 256
    pooled = rng.standard_normal((1, 2, n_q, n_kv // 128)).astype(np.float32)
    pooled[0, 1, :, :] = np.round(pooled[0, 1] * 2)        # ties in the second group
    check(pooled, n_q, n_kv, 2, 16, name="8192 blocks")


def test_chunk_with_offset():
    rng = np.random.default_rng(3400)
    n_kv, n_q, off = 50000, 777, 30001
    pooled = rng.standard_normal((1, 1, n_q, -(-n_kv // 128))).astype(np.float32)
    check(pooled, n_q, n_kv, 1, 16, q_offset=off, name="chunk")


# Rows of 1000 blocks (up to 16 keys per lane), an odd number of rows and
# three values of k around 32 selected blocks, with ties in one group.
@pytest.mark.parametrize("k", [16, 33, 34])
def test_rows_up_to_1024_blocks(k):
    rng = np.random.default_rng(3500 + k)
    n_kv, n_q = 128 * 1000, 333
    pooled = rng.standard_normal((1, 2, n_q, n_kv // 128)).astype(np.float32)
    pooled[0, 1] = np.round(pooled[0, 1] * 2)  # ties in the second group
    check(pooled, n_q, n_kv, 2, k, name=f"1000 blocks, k={k}")


def test_periodic_long_rows_take_the_exact_path():
    """As test_periodic_rows_take_the_exact_path, with 1000-block rows."""
    n_kv, n_q = 128 * 1000, 201
    t = np.arange(n_kv // 128)
    row = -(t % 64).astype(np.float32)
    pooled = np.broadcast_to(row, (1, 1, n_q, n_kv // 128)).copy()
    check(pooled, n_q, n_kv, 1, 16, name="periodic, 1000 blocks")


# Row lengths for every register width of the kernel (4, 32 and 64 keys per
# lane) and past 8192 blocks, where each pass re-reads the row.
@pytest.mark.parametrize("n_blk,n_q", [(200, 700), (1500, 301), (3000, 257), (9000, 64)])
def test_every_row_width(n_blk, n_q):
    rng = np.random.default_rng(3600 + n_blk)
    n_kv = 128 * n_blk - 77
    pooled = rng.standard_normal((1, 2, n_q, n_blk)).astype(np.float32) * 10
    pooled[0, 1] = np.round(pooled[0, 1])   # ties in the second group
    check(pooled, n_q, n_kv, 2, 16, name=f"{n_blk} blocks")


def test_ties_at_the_threshold():
    """The ten best scores are distinct and twenty blocks tie for the next
    place: the five lowest-indexed of the tied blocks are taken."""
    rng = np.random.default_rng(3700)
    n_q, n_blk = 256, 700
    n_kv = 128 * n_blk - 50          # positions from 128 * (n_blk - 3) + 78: at least n_blk - 3 candidates
    pooled = -rng.random((1, 1, n_q, n_blk)).astype(np.float32)
    for r in range(n_q):
        perm = rng.permutation(n_blk - 3)
        pooled[0, 0, r, perm[:10]] = 100.0 + np.arange(10)
        pooled[0, 0, r, perm[10:30]] = 50.0
    check(pooled, n_q, n_kv, 1, 16, name="threshold ties")


# Rows of 2049 .. 8192 blocks are selected by a workgroup of eight waves, 1024
# blocks each.  In one 5000-block launch: rows whose candidates end inside the
# first wave (a few blocks, or hundreds), across the first wave boundary and in
# later waves; with negative scores (the masked path), k of 1 (the local block
# alone), 2, 40 and 64, and lane-periodic scores (the exact search, which one
# wave streams).
WG_CASES = ["random", "negative", "k40", "periodic", "k1", "k2", "k64"]


@pytest.mark.parametrize("case", WG_CASES)
def test_workgroup_rows(case):
    rng = np.random.default_rng(3800 + WG_CASES.index(case))
    n_blk, n_q = 5000, 192
    n_kv = 128 * n_blk
    k = int(case[1:]) if case[0] == "k" else 16
    for off_blk in (16, 900, 1024, 3000, 4800):
        off = 128 * off_blk - 37
        if case == "periodic":
            row = -(np.arange(n_blk) % 64).astype(np.float32)
            pooled = np.broadcast_to(row, (1, 2, n_q, n_blk)).copy()
        else:
            pooled = rng.standard_normal((1, 2, n_q, n_blk)).astype(np.float32) * 10
            pooled[0, 1] = np.round(pooled[0, 1])   # ties in the second group
            if case == "negative":
                pooled = -np.abs(pooled) - 1.0
        check(pooled, n_q, n_kv, 2, k, q_offset=off, name=f"workgroup rows, {case}, from block {off_blk}")


# (queries, cache length) per sequence; the longest cache sets the row width:
# 469 blocks (8 keys per lane), 1016 (16), 1954 (32), 5469 (the workgroup path)
VARLEN_SEQS = {
    "per8": [(60, 60000), (20, 33000), (2, 130)],
    "per16": [(90, 130000), (41, 60000), (0, 5000), (3, 400)],
    "per32": [(70, 250000), (33, 131000), (5, 900)],
    "workgroup": [(100, 300000), (57, 700000), (0, 5000), (3, 400)],
}


@pytest.mark.parametrize("width", list(VARLEN_SEQS))
def test_varlen_long_rows(width):
    """msa_block_topk_v (the variable-length instantiations) on long caches:
    every sequence's rows equal the oracle's selection, and rows past a
    sequence's queries stay untouched."""
    import torch
    seqs = VARLEN_SEQS[width]
    B, h_kv, k = len(seqs), 2, 16
    qo = [q for q, _ in seqs]
    kv = [c for _, c in seqs]
    p = msa.Problem.make(B, max(qo), max(kv), 8 * h_kv, h_kv, topk=k)
    say(f"[gpu] top-k varlen long rows: seqs={seqs} n_blk={p.n_blk}")
    rng = np.random.default_rng(3900 + list(VARLEN_SEQS).index(width))
    pooled_np = (rng.standard_normal((B, h_kv, max(qo), p.n_blk)) * 10).astype(np.float32)
    pooled_np[:, 1] = np.round(pooled_np[:, 1])  # ties in the second group
    i32 = lambda a: torch.tensor(a, dtype=torch.int32, device="cuda")
    starts = np.concatenate([[0], np.cumsum(qo)[:-1]]).astype(int)
    vl = msa.Varlen.make(qo_lens=i32(qo), kv_lens=i32(kv), q_starts=i32(starts.tolist()), total_q=int(sum(qo)))
    bidx = torch.full((B, h_kv, max(qo), k), -77, dtype=torch.int32, device="cuda")
    msa.block_topk(p, torch.from_numpy(pooled_np).cuda(), bidx, varlen=vl)
    got = bidx.cpu().numpy()
    for b, (q_b, kv_b) in enumerate(seqs):
        assert (got[b, :, q_b:] == -77).all()
        if q_b == 0:
            continue
        pos = kv_b - q_b + np.arange(q_b)
        vis = np.arange(p.n_blk)[None, :] <= (pos // 128)[:, None]
        for g in range(h_kv):
            ref = oracle.select(np.where(vis, pooled_np[b, g, :q_b].astype(np.float64), np.nan), pos, 128, k)
            bad = np.nonzero(np.any(ref != got[b, g, :q_b], axis=1))[0]
            assert bad.size == 0, f"sequence {b} group {g} rows {bad[:5]}"
