"""GPU parity of variable-length batches and paged caches (the msa_*_v calls).

Each sequence of a batch is its own seeded workload (its own lengths); the
test packs the query-side tensors by row, lays the caches out either
contiguously (padded to the longest) or as a shuffled page pool addressed
through a page table, runs the HIP path through the C ABI and compares every
sequence with the fp64 oracle run on that sequence alone.  Pool and padding
memory the kernels must not use is filled with large values, so a read that
escapes the causal mask or a sequence's pages shows up in the outputs.
"""
import numpy as np
import pytest

import block_sparse_long_qk_amd as msa
import synth
from gpu_helpers import Stats, check_rows, problem, say

pytestmark = pytest.mark.gpu

# (name, h_q, h_kv, d_idx, k, [(qo_len, kv_len) per sequence])
CASES = [
    # prefill, a chunk, a decode row and a sequence without queries in one batch
    ("mix_prefill", 16, 2, 128, 16, [(3000, 3000), (257, 1500), (1, 4200), (640, 9000), (0, 300)]),
    # decode-shaped: at most 4 query rows per sequence (query-outer attention, streaming index)
    ("mix_decode", 16, 2, 128, 16, [(1, 5000), (3, 700), (1, 9000), (2, 128), (1, 1)]),
    # index dim 64, one KV head, small k, ragged caches
    ("mix_dimx64", 4, 1, 64, 8, [(500, 900), (1200, 1200), (77, 77)]),
    # FP8 (E4M3) index inputs, prefill and decode rows in one batch
    ("mix_fp8", 16, 2, 128, 16, [(2000, 2500), (1, 6000), (0, 10), (130, 130)], "fp8"),
    # FP8 (E4M3) K and V caches, bf16 index inputs
    ("mix_kv8", 16, 2, 128, 16, [(2000, 2500), (1, 6000), (0, 10), (130, 130), (3, 700)], "bf16", "fp8"),
]
SENTINEL_IDX = -77
SENTINEL_LSE = 12345.0


def _build(case, paged: bool, seed0: int):
    import torch
    name, h_q, h_kv, d_idx, k, seqs = case[:6]
    dtype = case[6] if len(case) > 6 else "bf16"
    kv_dtype = case[7] if len(case) > 7 else "bf16"
    B = len(seqs)
    ws = [synth.Workload(f"{name}_{b}", 1, max(qo, 1), kv, h_q, h_kv, index_dim=d_idx, topk=k, seed=seed0 + b,
                         index_dtype=dtype, kv_dtype=kv_dtype)
          for b, (qo, kv) in enumerate(seqs)]
    xs = [synth.device_inputs(w) for w in ws]
    qo_l = [qo for qo, _ in seqs]
    kv_l = [kv for _, kv in seqs]
    max_q, max_kv = max(max(qo_l), 1), max(kv_l)
    starts = np.concatenate([[0], np.cumsum(qo_l)[:-1]]).astype(np.int32)
    total_q = int(sum(qo_l))
    dev = xs[0]["q"].device
    big = 1.0e4
    ik_dtype = xs[0]["ik"].dtype

    def filled_index(shape):
        # memory the index kernels must not read: large values (E4M3: 448, code 0x7E)
        if ik_dtype == torch.uint8:
            return torch.full(shape, 0x7E, dtype=torch.uint8, device=dev)
        return torch.full(shape, big, dtype=torch.bfloat16, device=dev)

    def filled_kv(shape):
        # cache memory outside the sequences: large values (E4M3: 448, code 0x7E)
        if kv_dtype == "fp8":
            return torch.full(shape, 0x7E, dtype=torch.uint8, device=dev)
        return torch.full(shape, big, dtype=torch.bfloat16, device=dev)

    def pack(key):
        parts = [x[key][0, :qo] for x, qo in zip(xs, qo_l) if qo > 0]
        return torch.cat(parts).contiguous()

    q, iq = pack("q"), pack("iq")
    bk, d = 128, 128
    n_blk = [-(-kv // bk) for kv in kv_l]
    pps = -(-max_kv // bk)
    if paged:
        num_pages = sum(n_blk) + 3
        perm = np.random.default_rng(seed0).permutation(num_pages)
        table = np.zeros((B, pps), np.int32)
        at = 0
        for b in range(B):
            table[b, :n_blk[b]] = perm[at:at + n_blk[b]]
            table[b, n_blk[b]:] = perm[-1]     # never read: past the sequence's blocks
            at += n_blk[b]
        kp = filled_kv((num_pages, h_kv, bk, d))
        vp = filled_kv((num_pages, h_kv, bk, d))
        ikp = filled_index((num_pages, bk, d_idx))
        for b, x in enumerate(xs):
            for t in range(n_blk[b]):
                j0, j1 = t * bk, min((t + 1) * bk, kv_l[b])
                pg = int(table[b, t])
                kp[pg, :, :j1 - j0] = x["k"][0, :, j0:j1]
                vp[pg, :, :j1 - j0] = x["v"][0, :, j0:j1]
                ikp[pg, :j1 - j0] = x["ik"][0, j0:j1]
        table_t = torch.from_numpy(table).to(dev)
        k_in, v_in, ik_in = kp, vp, ikp
    else:
        num_pages, table_t = 0, None
        k_in = filled_kv((B, h_kv, max_kv, d))
        v_in = filled_kv((B, h_kv, max_kv, d))
        ik_in = filled_index((B, max_kv, d_idx))
        for b, x in enumerate(xs):
            k_in[b, :, :kv_l[b]] = x["k"][0]
            v_in[b, :, :kv_l[b]] = x["v"][0]
            ik_in[b, :kv_l[b]] = x["ik"][0]
    i32 = lambda a: torch.tensor(a, dtype=torch.int32, device=dev)
    vl = msa.Varlen.make(qo_lens=i32(qo_l), kv_lens=i32(kv_l), q_starts=i32(starts.tolist()), total_q=total_q,
                         page_table=table_t, num_pages=num_pages)
    p = msa.Problem.make(B, max_q, max_kv, h_q, h_kv, 128, d_idx, bk, k,
                         index_dtype=msa.DTYPE_FP8_E4M3 if dtype == "fp8" else msa.DTYPE_BF16,
                         kv_dtype=msa.DTYPE_FP8_E4M3 if kv_dtype == "fp8" else msa.DTYPE_BF16)
    return ws, xs, vl, p, dict(q=q, iq=iq, k=k_in, v=v_in, ik=ik_in), qo_l, starts, total_q


def _run(p, vl, x, total_q):
    import torch
    dev = x["q"].device
    B, h_q, h_kv, max_q, k = p.batch, p.h_q, p.h_kv, p.n_q, p.topk
    pooled = torch.empty((B, h_kv, max_q, p.n_blk), dtype=torch.float32, device=dev)
    bidx = torch.full((B, h_kv, max_q, k), SENTINEL_IDX, dtype=torch.int32, device=dev)
    out = torch.empty((total_q, h_q, 128), dtype=torch.bfloat16, device=dev)
    lse = torch.full((B, h_q, max_q), SENTINEL_LSE, dtype=torch.float32, device=dev)
    ws = torch.empty(max(msa.workspace_size(p, msa.OP_SPARSE_ATTN), 256), dtype=torch.uint8, device=dev)
    msa.index_scores(p, x["iq"], x["ik"], pooled, varlen=vl)
    msa.block_topk(p, pooled, bidx, varlen=vl)
    msa.sparse_attn_fwd(p, x["q"], x["k"], x["v"], bidx, out, lse, ws, varlen=vl)
    wf = torch.empty(max(msa.workspace_size(p, msa.OP_FORWARD), 256), dtype=torch.uint8, device=dev)
    fb = torch.full_like(bidx, SENTINEL_IDX)
    fo = torch.empty_like(out)
    fl = torch.full_like(lse, SENTINEL_LSE)
    msa.forward(p, x["q"], x["k"], x["v"], x["iq"], x["ik"], fo, fb, fl, wf, varlen=vl)
    torch.cuda.synchronize()
    return pooled, bidx, out, lse, (fo, fb, fl)


@pytest.mark.parametrize("paged", [True, False], ids=["paged", "contiguous"])
@pytest.mark.parametrize("ci", range(len(CASES)), ids=[c[0] for c in CASES])
def test_varlen_matches_oracle_per_sequence(ci, paged):
    import torch
    case = CASES[ci]
    say(f"[gpu] varlen {case[0]} paged={paged} seqs={case[5]}")
    ws, xs, vl, p, x, qo_l, starts, total_q = _build(case, paged, seed0=3100 + 10 * ci)
    pooled, bidx, out, lse, (fo, fb, fl) = _run(p, vl, x, total_q)
    # msa_forward equals the three calls
    assert torch.equal(fb, bidx)
    assert torch.equal(fo.view(torch.int16), out.view(torch.int16))
    assert torch.equal(fl, lse)
    st = Stats()
    for b, w in enumerate(ws):
        qo = qo_l[b]
        # rows past a sequence's queries are left untouched
        assert bool((bidx[b, :, qo:] == SENTINEL_IDX).all())
        assert bool((lse[b, :, qo:] == SENTINEL_LSE).all())
        if qo == 0:
            continue
        res = {"pooled": pooled[b:b + 1], "block_idx": bidx[b:b + 1],
               "out": out[int(starts[b]):int(starts[b]) + qo].unsqueeze(0), "lse": lse[b:b + 1]}
        rows = np.arange(qo) if qo <= 700 else np.unique(np.concatenate(
            [np.arange(0, 130), np.arange(qo - 130, qo), np.random.default_rng(b).integers(0, qo, 200)]))
        for g in range(w.h_kv):
            check_rows(w, res, 0, g, rows, st)
    st.check()


def test_varlen_uniform_equals_plain_call():
    """A Varlen that only restates the uniform layout gives the plain call's bits."""
    import torch
    w = synth.Workload("varlen_uniform", 2, 700, 900, 8, 2, topk=6, seed=3190)
    x = synth.device_inputs(w)
    p = msa.Problem.make(w.batch, w.n_q, w.n_kv, w.h_q, w.h_kv, 128, 128, 128, w.topk)
    dev = x["q"].device
    i32 = lambda a: torch.tensor(a, dtype=torch.int32, device=dev)
    vl = msa.Varlen.make(qo_lens=i32([w.n_q] * 2), kv_lens=i32([w.n_kv] * 2), q_starts=i32([0, w.n_q]),
                         total_q=2 * w.n_q)
    outs = []
    for v in (None, vl):
        f = msa.alloc_outputs(p, dev)
        msa.forward(p, x["q"], x["k"], x["v"], x["iq"], x["ik"], f["out"], f["block_idx"], f["lse"], f["workspace"],
                    varlen=v)
        torch.cuda.synchronize()
        outs.append(f)
    assert torch.equal(outs[0]["block_idx"], outs[1]["block_idx"])
    assert torch.equal(outs[0]["out"].view(torch.int16), outs[1]["out"].view(torch.int16))
    assert torch.equal(outs[0]["lse"], outs[1]["lse"])


def test_paged_128k_equals_contiguous():
    """The benchmarked 128K prefill read from a page pool (k/v
    [pages][h_kv][Bk][d], index_k [pages][Bk][d_idx], pages in a seeded random
    order) gives the bits of the contiguous call, which test_gpu_parity checks
    against the oracle at this size."""
    import torch
    w = synth.WORKLOADS["prefill_128k"]
    say(f"[gpu] paged {w.name} against contiguous")
    x = synth.device_inputs(w)
    dev = x["q"].device
    p = problem(w)
    f = msa.alloc_outputs(p, dev)
    msa.forward(p, x["q"], x["k"], x["v"], x["iq"], x["ik"], f["out"], f["block_idx"], f["lse"], f["workspace"])
    torch.cuda.synchronize()
    ref = {key: f[key].clone() for key in ("out", "block_idx", "lse")}
    B, hk, bk, d, di, pps = w.batch, w.h_kv, w.block_size, w.head_dim, w.index_dim, w.n_blk
    assert w.n_kv == pps * bk
    perm = torch.from_numpy(np.random.default_rng(w.seed).permutation(B * pps)).to(dev)
    pool = {}
    for name, page_shape in (("k", (hk, bk, d)), ("v", (hk, bk, d)), ("ik", (bk, di))):
        dst = torch.empty((B * pps,) + page_shape, dtype=torch.bfloat16, device=dev)
        for b in range(B):
            src = x[name][b].view(hk, pps, bk, d).transpose(0, 1) if name != "ik" else x[name][b].view(pps, bk, di)
            dst.index_copy_(0, perm[b * pps:(b + 1) * pps], src)
        pool[name] = dst
    i32 = lambda a: a.to(torch.int32).contiguous()
    vl = msa.Varlen.make(qo_lens=i32(torch.full((B,), w.n_q, device=dev)),
                         kv_lens=i32(torch.full((B,), w.n_kv, device=dev)),
                         q_starts=i32(torch.arange(B, device=dev) * w.n_q), total_q=B * w.n_q,
                         page_table=i32(perm.view(B, pps)), num_pages=B * pps)
    for key in ("out", "block_idx", "lse"):
        f[key].fill_(-1)
    msa.forward(p, x["q"], pool["k"], pool["v"], x["iq"], pool["ik"], f["out"], f["block_idx"], f["lse"],
                f["workspace"], varlen=vl)
    torch.cuda.synchronize()
    assert torch.equal(ref["block_idx"], f["block_idx"])
    assert torch.equal(ref["lse"], f["lse"])
    assert torch.equal(ref["out"].view(torch.int16), f["out"].view(torch.int16))
    del x, f, ref, pool
    torch.cuda.empty_cache()
