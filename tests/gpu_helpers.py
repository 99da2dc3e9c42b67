"""Helpers of the GPU parity tests: run the HIP path through the C ABI and
compare it with the fp64 oracle on the same seeded inputs.

The tolerances are the ones the task fixes: block indices bit-exact where the
gap between the (k-1)-th and k-th best non-local pooled score exceeds 1e-3
(relative), epsilon-valid inside that gap; outputs within max |d| <= 1e-2 and
mean |d| <= 1e-3 of the oracle run on the same block set.  Pooled scores must
lie within the fp32 summation bound 2 * d_idx * 2^-24 * max_j sum_c |iq_c ik_jc|
(bf16 products are exact in fp32; any accumulation order), plus, for E4M3
index inputs, the run truncation of the E4M3 MFMA (see tau_pool).
"""
from __future__ import annotations

import sys

import numpy as np

import block_sparse_long_qk_amd as msa
import oracle
import synth
from oracle import accept

OUT_MAX_ABS = 1e-2
OUT_MEAN_ABS = 1e-3
LSE_ABS = 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def problem(w: synth.Workload) -> msa.Problem:
    dt = msa.DTYPE_FP8_E4M3 if w.index_dtype == "fp8" else msa.DTYPE_BF16
    kt = msa.DTYPE_FP8_E4M3 if w.kv_dtype == "fp8" else msa.DTYPE_BF16
    return msa.Problem.make(w.batch, w.n_q, w.n_kv, w.h_q, w.h_kv, w.head_dim, w.index_dim, w.block_size, w.topk,
                            w.q_offset, w.scale, index_dtype=dt, kv_dtype=kt)


def bf16_np(t) -> np.ndarray:
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def run_gpu(w: synth.Workload, inputs=None, with_forward=True, stream=None) -> dict:
    """Run the three stages (and the fused forward) on device inputs."""
    import torch
    say(f"[gpu] {w.name}: B={w.batch} n_q={w.n_q} n_kv={w.n_kv} h={w.h_q}/{w.h_kv} d_idx={w.index_dim} k={w.topk}")
    x = synth.device_inputs(w) if inputs is None else inputs
    p = problem(w)
    dev = x["q"].device
    pooled = torch.empty((w.batch, w.h_kv, w.n_q, w.n_blk), dtype=torch.float32, device=dev)
    bidx = torch.empty((w.batch, w.h_kv, w.n_q, w.topk), dtype=torch.int32, device=dev)
    out = torch.empty((w.batch, w.n_q, w.h_q, w.head_dim), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.batch, w.h_q, w.n_q), dtype=torch.float32, device=dev)
    ws = torch.empty(max(msa.workspace_size(p, msa.OP_SPARSE_ATTN), 256), dtype=torch.uint8, device=dev)
    msa.index_scores(p, x["iq"], x["ik"], pooled, stream)
    msa.block_topk(p, pooled, bidx, stream)
    msa.sparse_attn_fwd(p, x["q"], x["k"], x["v"], bidx, out, lse, ws, stream=stream)
    torch.cuda.synchronize()
    del ws
    res = {"inputs": x, "pooled": pooled, "block_idx": bidx, "out": out, "lse": lse}
    if with_forward:
        f = msa.alloc_outputs(p, dev)
        msa.forward(p, x["q"], x["k"], x["v"], x["iq"], x["ik"], f["out"], f["block_idx"], f["lse"], f["workspace"],
                    stream=stream)
        torch.cuda.synchronize()
        res["fwd"] = {k: f[k] for k in ("out", "block_idx", "lse")}
        del f
    return res


def index_values(x) -> np.ndarray:
    """Index inputs as fp64 values: bf16 bits (uint16) or E4M3 codes (uint8)."""
    x = np.asarray(x)
    return oracle.e4m3_decode(x) if x.dtype == np.uint8 else synth.bf16_to_f32(x).astype(np.float64)


# The gfx950 E4M3 MFMA sums each run of 8 consecutive k-elements of a lane's
# operand in a fixed-point adder aligned to the run's largest product, keeping
# 13 bits below it (smaller products truncated toward zero), and accumulates
# the run sums in fp32 (measured: a product 2^-14 or less relative to the
# largest of its run is dropped, one in another run is kept exactly).  Per
# score that adds at most 7 * 2^-13 * max|p| per run; the bound below takes
# 2^-12 (a factor 2 of margin) and bounds max|p| over a run by the product of
# the runs' largest |iq| and |ik| (runs = 8 consecutive index dims).
E4M3_RUN = 8
E4M3_RUN_ERR = 7 * 2.0 ** -12


def tau_pool(iq_rows, ik, pos, bk):
    """Per (row, block) bound on |pooled_gpu - pooled_exact|: the fp32
    summation bound 2 * d_idx * 2^-24 * sum|p| (bf16 and E4M3 products are exact
    in fp32), plus the run truncation of the E4M3 MFMA for E4M3 inputs."""
    a = np.abs(index_values(iq_rows))
    b = np.abs(index_values(ik))
    s = 2.0 * iq_rows.shape[1] * 2.0 ** -24 * (a @ b.T)    # [n, n_kv]
    if np.asarray(iq_rows).dtype == np.uint8:
        ra = a.reshape(a.shape[0], -1, E4M3_RUN).max(axis=2)
        rb = b.reshape(b.shape[0], -1, E4M3_RUN).max(axis=2)
        s = s + E4M3_RUN_ERR * (ra @ rb.T)
    n_kv = ik.shape[0]
    n_blk = -(-n_kv // bk)
    pad = np.full((len(pos), n_blk * bk), -np.inf)
    pad[:, :n_kv] = s
    pad[np.arange(n_blk * bk)[None, :] > np.asarray(pos)[:, None]] = -np.inf
    return pad.reshape(len(pos), n_blk, bk).max(axis=2)


class Stats:
    def __init__(self):
        self.max_abs = 0.0
        self.sum_abs = 0.0
        self.n = 0
        self.lse_max = 0.0
        self.verdicts = {"exact": 0, "eps": 0, "FAIL": 0}

    def add_out(self, got, ref):
        d = np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))
        self.max_abs = max(self.max_abs, float(d.max()) if d.size else 0.0)
        self.sum_abs += float(d.sum())
        self.n += d.size

    def add_lse(self, got, ref):
        d = np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))
        self.lse_max = max(self.lse_max, float(d.max()) if d.size else 0.0)

    @property
    def mean_abs(self):
        return self.sum_abs / max(self.n, 1)

    def check(self):
        say(f"    out max|d|={self.max_abs:.3e} mean|d|={self.mean_abs:.3e} lse max|d|={self.lse_max:.3e} "
            f"indices {self.verdicts}")
        assert self.verdicts["FAIL"] == 0
        assert self.max_abs <= OUT_MAX_ABS
        assert self.mean_abs <= OUT_MEAN_ABS
        assert self.lse_max <= LSE_ABS


def check_rows(w: synth.Workload, res: dict, b: int, g: int, rows, stats: Stats, plant=None):
    """Compare the GPU result of some query rows of one (sequence, group)."""
    rows = np.asarray(rows, dtype=np.int64)
    G, bk, k = w.group, w.block_size, w.topk
    x = oracle.inputs_for_rows(w, b, g, rows, plant)
    pos = x["pos"]
    local = pos // bk
    # pooled scores within the summation bound (visible part only)
    pooled_ref = oracle.pool_for(w, x["iq"], pos, x["ik"])
    nb = pooled_ref.shape[1]
    idx = torch_index(rows)
    pooled_gpu = res["pooled"][b, g].index_select(0, idx).cpu().numpy()[:, :nb].astype(np.float64)
    tau = tau_pool(x["iq"], x["ik"], pos, bk)
    vis = np.arange(nb)[None, :] <= local[:, None]
    err = np.where(vis, np.abs(pooled_gpu - np.nan_to_num(pooled_ref)), 0.0)
    assert np.all(err <= np.where(vis, tau, 0.0) + 1e-30), f"pooled beyond bound: {np.max(err / (tau + 1e-30))}"
    # the GPU top-k on its own fp32 scores is the oracle's selection on those values, bit for bit
    sel_gpu = res["block_idx"][b, g].index_select(0, idx).cpu().numpy()
    pg = np.where(vis, pooled_gpu, np.nan)
    assert np.array_equal(oracle.select(pg, pos, bk, k), sel_gpu), "top-k differs on identical fp32 input"
    # indices against the oracle's own fp64 selection (gap rule)
    sel_ref = oracle.select(pooled_ref, pos, bk, k)
    for v in accept.check_indices(sel_gpu, sel_ref, pooled_ref, local, k):
        stats.verdicts[v] += 1
    # attention on the GPU's block set
    K, V = oracle.kv_for_blocks(w, b, g, sel_gpu)
    out_ref, lse_ref = oracle.attend(x["q"], pos, sel_gpu, K, V, bk, w.scale)
    out_gpu = res["out"][b].index_select(0, idx)[:, g * G:(g + 1) * G, :].float().cpu().numpy()
    stats.add_out(out_gpu, out_ref)
    lse_gpu = res["lse"][b, g * G:(g + 1) * G].index_select(1, idx).cpu().numpy().T
    stats.add_lse(lse_gpu, lse_ref)


def torch_index(rows):
    import torch
    return torch.from_numpy(np.asarray(rows, dtype=np.int64)).cuda()


def check_forward_matches_stages(res: dict):
    import torch
    f = res["fwd"]
    assert torch.equal(f["block_idx"], res["block_idx"])
    assert torch.equal(f["out"].view(torch.int16), res["out"].view(torch.int16))
    assert torch.equal(f["lse"], res["lse"])


def sample_rows(w: synth.Workload, n_random: int, seed: int, whole_blocks: int = 0):
    """Edge rows (first/last, block boundaries, the k*Bk threshold) plus random rows,
    plus every row of a few random query blocks."""
    rng = np.random.default_rng(seed)
    bk, off, nq = w.block_size, w.offset, w.n_q
    cand = {0, nq - 1, min(nq - 1, 1), min(nq - 1, bk - 1 - off % bk)}
    for p in (bk - 1, bk, w.topk * bk - 1, w.topk * bk, w.topk * bk + 1, 2047, 2048, w.n_kv - bk, w.n_kv - 1):
        if off <= p < off + nq:
            cand.add(p - off)
    cand.update(rng.integers(0, nq, size=n_random).tolist())
    for _ in range(whole_blocks):
        s = int(rng.integers(0, max(1, nq // bk))) * bk
        cand.update(range(s, min(s + bk, nq)))
    return np.array(sorted(cand), dtype=np.int64)
