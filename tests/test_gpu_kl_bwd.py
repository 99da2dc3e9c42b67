"""GPU parity of the KL backward into the Index Branch (msa_index_kl_bwd)
against the fp64 oracle (oracle_kl_bwd, pinned to torch autograd with the
teacher detached).

The forward pass and the KL pass run on the GPU (block_idx, lse, lse_index);
the KL backward then takes them through the C ABI.  Small cases compare
d_index_q and d_index_k element by element with the oracle over every row of
each group (the GPU's own selection; d_index_k is the sum of the groups'
contributions, since the index keys are shared); one case takes random row
weights dkl.  The 32K and 128K workloads compare d_index_q on sampled rows
and d_index_k of one key block against the oracle over every row (of every
group) that attends it, and check the sum rule: every row's g_j = w (s_j - t_j) sums to zero over T (student
and teacher are both distributions over T), so sum_j d_index_k[j] = 0.

Tolerance: g enters the MFMA as bf16 (relative error 2^-9), the index inputs
are exact bf16, sums run in fp32 and the results (and the d_index_q partials)
are rounded to bf16: an element is off by about 2^-8 of the magnitude of the
terms it sums.  The bound is the one of the attention backward: 2e-2 of the
tensor's largest |value| for every element, 2e-3 of it on average.

The stored-teacher pair (msa_index_kl_teacher, msa_index_kl_bwd_teacher): the
KL pass with the teacher kept writes the same kl and lse_index bits as
msa_index_kl; every stored weight of every used (row, slot) matches the
oracle's teacher (oracle_kl_teacher) to fp16 rounding (2^-11 relative) plus
the fp32 lse's error, and keys outside T hold 0; the backward from the stored
teacher meets the same bound against oracle_kl_bwd as msa_index_kl_bwd.
"""
import numpy as np
import pytest

import block_sparse_long_qk_amd as msa
import oracle
import synth
from gpu_helpers import problem, run_gpu, sample_rows, say

pytestmark = pytest.mark.gpu

GRAD_MAX_REL, GRAD_MEAN_REL = 2e-2, 2e-3

CASES = [
    synth.Workload("klb_g8", 1, 2048, 2048, 16, 2, topk=8, seed=2701),
    synth.Workload("klb_g4_ragged_dimx64", 2, 1000, 1000, 8, 2, index_dim=64, topk=4, seed=2702),
    synth.Workload("klb_g16_chunk", 1, 300, 1000, 32, 2, topk=4, q_offset=700, seed=2703),
    synth.Workload("klb_g32", 1, 1536, 1536, 32, 1, topk=5, seed=2704),
    synth.Workload("klb_decode", 3, 1, 5000, 16, 2, topk=8, seed=2705),
    synth.Workload("klb_one_token", 2, 1, 1, 16, 2, seed=2706),
]
WEIGHTED = {"klb_g4_ragged_dimx64"}


def run_kl_bwd(w, res, dkl=None):
    import torch
    p = problem(w)
    x = res["inputs"]
    kl = torch.empty((w.batch, w.h_kv, w.n_q), dtype=torch.float32, device="cuda")
    lse_index = torch.full_like(kl, float("nan"))
    ws = torch.empty(max(msa.workspace_size(p, msa.OP_INDEX_KL), 256), dtype=torch.uint8, device="cuda")
    msa.index_kl(p, x["q"], x["k"], x["iq"], x["ik"], res["block_idx"], res["lse"], kl, ws, lse_index=lse_index)
    del ws
    d_iq = torch.full_like(x["iq"], float("nan"))  # every element must be written
    d_ik = torch.full_like(x["ik"], float("nan"))
    ws = torch.empty(msa.workspace_size(p, msa.OP_INDEX_KL_BWD), dtype=torch.uint8, device="cuda")
    msa.index_kl_bwd(p, x["q"], x["k"], x["iq"], x["ik"], res["block_idx"], res["lse"], lse_index, d_iq, d_ik,
                     dkl=dkl, workspace=ws)
    torch.cuda.synchronize()
    return lse_index, d_iq, d_ik


def as_float(t):
    import torch
    return t.view(torch.bfloat16).float().cpu().numpy()


def close(name, got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    # the bound is relative to the tensor's largest |value|, floored at 1e-3 (three
    # orders below these gradients' size) for gradients that vanish exactly, as
    # with a single visible token (its weight is 1 and dS = 0)
    scale = max(np.abs(ref).max(), 1e-3)
    err = np.abs(got - ref)
    say(f"    {name}: max |d| {err.max():.3e} (rel {err.max() / scale:.2e}), mean rel {err.mean() / scale:.2e}")
    assert np.all(np.isfinite(got)), name
    assert err.max() <= GRAD_MAX_REL * scale and err.mean() <= GRAD_MEAN_REL * scale, name


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_kl_backward_matches_oracle(w):
    import torch
    say(f"[gpu] kl backward {w.name}: B={w.batch} n_q={w.n_q} n_kv={w.n_kv} h={w.h_q}/{w.h_kv} "
        f"d_idx={w.index_dim} k={w.topk}")
    res = run_gpu(w, with_forward=False)
    dkl = None
    if w.name in WEIGHTED:
        gen = torch.Generator().manual_seed(w.seed)
        dkl = (torch.rand((w.batch, w.h_kv, w.n_q), generator=gen) * 2 - 0.5).cuda()
    _, d_iq, d_ik = run_kl_bwd(w, res, dkl)
    rows = np.arange(w.n_q)
    for b in range(w.batch):
        ref_ik = None
        for g in range(w.h_kv):
            x = oracle.inputs_for_rows(w, b, g, rows)
            sel = res["block_idx"][b, g].cpu().numpy()
            K = synth.host_kv(w, "k", b, g, 0, w.n_kv)
            wr = None if dkl is None else dkl[b, g].double().cpu().numpy()
            r_iq, r_ik = oracle.kl_bwd(x["q"], x["pos"], sel, K, x["iq"], x["ik"], w.block_size, w.scale, wr)
            close(f"d_iq b{b} g{g}", as_float(d_iq[b][:, g]), r_iq)
            ref_ik = r_ik if ref_ik is None else ref_ik + r_ik
        got_ik = as_float(d_ik[b])
        n_seen = ref_ik.shape[0]
        close(f"d_ik b{b}", got_ik[:n_seen], ref_ik)
        assert np.all(got_ik[n_seen:] == 0.0), "keys past every row's position must get 0"


def check_block_dik(w, res, d_ik, t):
    """d_index_k of key block t, exactly: the index keys are shared by the
    groups, so the oracle runs over every row of every group whose block set
    holds t (the only rows whose gradients reach those keys) and the groups'
    contributions are added."""
    import torch
    j0, j1 = t * w.block_size, min((t + 1) * w.block_size, w.n_kv)
    ref = np.zeros((j1 - j0, w.index_dim))
    n_rows = 0
    for g in range(w.h_kv):
        sel_all = res["block_idx"][0, g].cpu().numpy()
        rows = np.nonzero((sel_all == t).any(axis=1))[0]
        assert len(rows) > 0
        n_rows += len(rows)
        x = oracle.inputs_for_rows(w, 0, g, rows)
        sel = sel_all[rows]
        K, _ = oracle.kv_for_blocks(w, 0, g, sel)
        _, r_ik = oracle.kl_bwd(x["q"], x["pos"], sel, K, x["iq"], x["ik"], w.block_size, w.scale)
        ref += r_ik[j0:j1]
    got = d_ik[0].view(torch.bfloat16)[j0:j1].float().cpu().numpy()
    close(f"d_ik block {t} ({n_rows} rows over the groups)", got, ref)


@pytest.mark.parametrize("name,n_rand", [("prefill_32k", 32), ("prefill_128k", 16)])
def test_kl_backward_full_size_sampled_and_sum_rule(name, n_rand):
    """At 32K and at the benchmarked 128K: d_index_q on sampled rows, d_index_k
    of one late key block exactly, and the sum rule over every key."""
    import torch
    w = synth.WORKLOADS[name]
    say(f"[gpu] kl backward {w.name}")
    res = run_gpu(w, with_forward=False)
    _, d_iq, d_ik = run_kl_bwd(w, res)
    rows = sample_rows(w, n_rand, seed=w.seed, whole_blocks=0)
    for g in range(w.h_kv):
        x = oracle.inputs_for_rows(w, 0, g, rows)
        sel = res["block_idx"][0, g].cpu().numpy()[rows]
        K, _ = oracle.kv_for_blocks(w, 0, g, sel)
        r_iq, _ = oracle.kl_bwd(x["q"], x["pos"], sel, K, x["iq"], x["ik"], w.block_size, w.scale)
        got = as_float(d_iq[0].index_select(0, torch.from_numpy(rows).cuda())[:, g])
        close(f"d_iq g{g}", got, r_iq)
    dik = d_ik[0].view(torch.bfloat16).float()
    total = dik.sum(dim=0)
    mag = dik.abs().sum(dim=0)
    say(f"    sum rule: max |sum_j d_ik_j| / sum_j |d_ik_j| = {(total.abs() / mag).max().item():.2e}")
    assert bool(torch.isfinite(dik).all())
    assert bool((total.abs() <= 1e-2 * mag).all())
    check_block_dik(w, res, d_ik, w.n_blk - 24)


def test_kl_backward_is_deterministic():
    """Two calls on the same inputs give the same bits (sorted plan bins, the
    groups' d_index_k shares added in group order)."""
    import torch
    w = synth.WORKLOADS["prefill_32k"]
    res = run_gpu(w, with_forward=False)
    _, a_iq, a_ik = run_kl_bwd(w, res)
    _, b_iq, b_ik = run_kl_bwd(w, res)
    assert torch.equal(a_iq.view(torch.int16), b_iq.view(torch.int16))
    assert torch.equal(a_ik.view(torch.int16), b_ik.view(torch.int16))


# ---------------------------------------------------------------- stored teacher
TEACHER_REL, TEACHER_ABS = 1e-3, 1e-7


def run_kl_teacher(w, res):
    import torch
    p = problem(w)
    x = res["inputs"]
    kl = torch.empty((w.batch, w.h_kv, w.n_q), dtype=torch.float32, device="cuda")
    lse_index = torch.full_like(kl, float("nan"))
    teacher = torch.full(msa.teacher_shape(p), float("nan"), dtype=torch.float16, device="cuda")
    ws = torch.empty(max(msa.workspace_size(p, msa.OP_INDEX_KL), 256), dtype=torch.uint8, device="cuda")
    msa.index_kl_teacher(p, x["q"], x["k"], x["iq"], x["ik"], res["block_idx"], res["lse"], kl, lse_index, teacher,
                         ws)
    torch.cuda.synchronize()
    return kl, lse_index, teacher


def run_kl_bwd_teacher(w, res, teacher, lse_index, dkl=None):
    import torch
    p = problem(w)
    x = res["inputs"]
    d_iq = torch.full_like(x["iq"], float("nan"))
    d_ik = torch.full_like(x["ik"], float("nan"))
    ws = torch.empty(msa.workspace_size(p, msa.OP_INDEX_KL_BWD), dtype=torch.uint8, device="cuda")
    msa.index_kl_bwd_teacher(p, x["iq"], x["ik"], res["block_idx"], teacher, lse_index, d_iq, d_ik, dkl=dkl,
                             workspace=ws)
    torch.cuda.synchronize()
    return d_iq, d_ik


def used_slots(sel_row, local, k):
    """Slots of a row the kernels use: listed non-local blocks (first of equal
    neighbours) and slot k for the local block."""
    out = [(s, int(t)) for s, t in enumerate(sel_row) if 0 <= t < local and (s == 0 or sel_row[s - 1] != t)]
    return out + [(k, local)]


def check_teacher(w, teacher_bg, ref, sel, rows):
    """teacher_bg [n_q, k+1, Bk] (fp32 of the stored fp16) against the oracle's
    dense teacher ref [len(rows), n_kv] over every used (row, slot)."""
    bk = w.block_size
    worst = 0.0
    for r, i in enumerate(rows):
        local = (w.offset + int(i)) // bk
        for s, t in used_slots(sel[i], local, w.topk):
            keys = t * bk + np.arange(bk)
            got = teacher_bg[i, s]
            inside = keys < w.n_kv
            want = np.zeros(bk)
            want[inside] = ref[r, keys[inside]]
            err = np.abs(got - want)
            assert np.all(np.isfinite(got)), (i, s)
            bad = np.nonzero(err > TEACHER_REL * want + TEACHER_ABS)[0]
            assert bad.size == 0, (int(i), s, int(t), [(int(j), float(got[j]), float(want[j])) for j in bad[:6]])
            worst = max(worst, float((err / (want + TEACHER_ABS)).max()))
    return worst


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_stored_teacher_and_its_backward_match_oracle(w):
    import torch
    say(f"[gpu] stored teacher {w.name}: B={w.batch} n_q={w.n_q} n_kv={w.n_kv} h={w.h_q}/{w.h_kv} "
        f"d_idx={w.index_dim} k={w.topk}")
    res = run_gpu(w, with_forward=False)
    lz0, _, _ = run_kl_bwd(w, res)
    kl, lse_index, teacher = run_kl_teacher(w, res)
    assert torch.equal(lse_index, lz0), "the teacher-keeping pass gives the same lse_index bits"
    dkl = None
    if w.name in WEIGHTED:
        gen = torch.Generator().manual_seed(w.seed)
        dkl = (torch.rand((w.batch, w.h_kv, w.n_q), generator=gen) * 2 - 0.5).cuda()
    d_iq, d_ik = run_kl_bwd_teacher(w, res, teacher, lse_index, dkl)
    tf = teacher.float().cpu().numpy()
    rows = np.arange(w.n_q)
    for b in range(w.batch):
        ref_ik = None
        for g in range(w.h_kv):
            x = oracle.inputs_for_rows(w, b, g, rows)
            sel = res["block_idx"][b, g].cpu().numpy()
            K = synth.host_kv(w, "k", b, g, 0, w.n_kv)
            ref_t = oracle.kl_teacher(x["q"], x["pos"], sel, K, w.block_size, w.scale)
            worst = check_teacher(w, tf[b, g], ref_t, sel, rows)
            say(f"    teacher b{b} g{g}: worst relative error {worst:.2e}")
            wr = None if dkl is None else dkl[b, g].double().cpu().numpy()
            r_iq, r_ik = oracle.kl_bwd(x["q"], x["pos"], sel, K, x["iq"], x["ik"], w.block_size, w.scale, wr)
            close(f"d_iq b{b} g{g}", as_float(d_iq[b][:, g]), r_iq)
            ref_ik = r_ik if ref_ik is None else ref_ik + r_ik
        got_ik = as_float(d_ik[b])
        n_seen = ref_ik.shape[0]
        close(f"d_ik b{b}", got_ik[:n_seen], ref_ik)
        assert np.all(got_ik[n_seen:] == 0.0), "keys past every row's position must get 0"


@pytest.mark.parametrize("name,n_rand", [("prefill_32k", 32), ("prefill_128k", 16)])
def test_stored_teacher_full_size_sampled_sum_rule_and_determinism(name, n_rand):
    import torch
    w = synth.WORKLOADS[name]
    say(f"[gpu] stored teacher {w.name}")
    res = run_gpu(w, with_forward=False)
    _, lse_index, teacher = run_kl_teacher(w, res)
    d_iq, d_ik = run_kl_bwd_teacher(w, res, teacher, lse_index)
    rows = sample_rows(w, n_rand, seed=w.seed + 1, whole_blocks=0)
    tf = teacher.float().cpu().numpy()
    for g in range(w.h_kv):
        x = oracle.inputs_for_rows(w, 0, g, rows)
        sel_all = res["block_idx"][0, g].cpu().numpy()
        sel = sel_all[rows]
        K, _ = oracle.kv_for_blocks(w, 0, g, sel)
        r_iq, _ = oracle.kl_bwd(x["q"], x["pos"], sel, K, x["iq"], x["ik"], w.block_size, w.scale)
        got = as_float(d_iq[0].index_select(0, torch.from_numpy(rows).cuda())[:, g])
        close(f"d_iq g{g}", got, r_iq)
        if g == 0:
            ref_t = oracle.kl_teacher(x["q"], x["pos"], sel, K, w.block_size, w.scale)
            worst = check_teacher(w, tf[0, g], ref_t, sel_all, rows)
            say(f"    teacher g0 (sampled rows): worst relative error {worst:.2e}")
    dik = d_ik[0].view(torch.bfloat16).float()
    total, mag = dik.sum(dim=0), dik.abs().sum(dim=0)
    say(f"    sum rule: max |sum_j d_ik_j| / sum_j |d_ik_j| = {(total.abs() / mag).max().item():.2e}")
    assert bool(torch.isfinite(dik).all())
    assert bool((total.abs() <= 1e-2 * mag).all())
    check_block_dik(w, res, d_ik, w.n_blk - 24)
    a_iq, a_ik = run_kl_bwd_teacher(w, res, teacher, lse_index)
    assert torch.equal(a_iq.view(torch.int16), d_iq.view(torch.int16))
    assert torch.equal(a_ik.view(torch.int16), d_ik.view(torch.int16))
