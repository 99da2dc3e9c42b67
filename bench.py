"""Benchmark of the MSA forward pass on one MI355X.

One step = one msa_forward call (index scores + block max-pool and block
top-k, gather plan, sparse attention, merge) over the 128K-token causal
prefill (batch 1, 64 query heads on 8 KV heads, head dim 128, index dim 128,
Bk 128, k 16), inputs seeded and synthetic, resident in HBM before timing
starts.  The timed steps go through msa_forward_marked, which records a HIP
event after each kernel on the launch stream, so every kernel's time in the
step is measured live.  Prints one JSON line: prefill tokens/s (the value),
step-time statistics, the roofline of the step's dominant kernel and a line per
kernel, a check that the timed block indices equal the staged calls', the
32K prefill and the 1M-context chunk as lines of their own, the 256K decode
step (64 sequences), cold-cache 4K and 32K steps, the same two headline steps
with the caches in a shuffled page pool, with FP8 index inputs and FP8 K/V,
the KL pass, both backward passes and dense mode at 128K, and the oracle's CPU
rate on a bounded sample of the same workload (with the host's description, a
single-thread run of the 4K workload and the extrapolated full-run time).
"""
import argparse
import hashlib
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
MAX_MARKS = 192                # events per marked step (overlapped passes mark ~100)

# HBM bytes per launch from rocprofv3 counter runs of the 128K step (FETCH_SIZE
# x2, calibrated on a 1 GiB copy, + WRITE_SIZE x1; see profiles/), with the
# sha256 (first 16 hex digits) of the sources the kernel was built from when
# they were taken.  A kernel whose sources have changed since reports null.
COUNTER_TRAFFIC = {
    # kernel name: (bytes per step, summed over the step's launches, {source file: sha16});
    # profiles/prefill_128k_decode_256k_counters.md
    "k_index_scores(top-k fused)": (3135016960, {"index_scores.hip": "d6c53c22822df47d", "common.h": "ecb32c13321b9a30"}),
    "k_attn_tiles": (59811840000, {"sparse_attn.hip": "531179aaf5e19eff", "fwd_tiles.h": "1f0a406284261b7e", "attn_tiles.h": "2f9107ca13d54488", "common.h": "ecb32c13321b9a30"}),
    "k_attn_local_merge": (31339520000, {"sparse_attn.hip": "531179aaf5e19eff", "fwd_tiles.h": "1f0a406284261b7e", "attn_tiles.h": "2f9107ca13d54488", "common.h": "ecb32c13321b9a30"}),
    "k_block_topk": (2285998080, {"block_topk.hip": "52d43fa6ee7deeff", "common.h": "ecb32c13321b9a30"}),
    "k_index_small": (4354646016, {"decode.hip": "6cb61b92818c32a7", "common.h": "ecb32c13321b9a30"}),
    "k_attn_rows": (575160320, {"decode.hip": "6cb61b92818c32a7", "common.h": "ecb32c13321b9a30"}),
}
COUNTER_WORKLOAD = {"k_index_small": "decode_256k", "k_attn_rows": "decode_256k"}  # the others: prefill_128k


def source_sha16(name):
    path = os.path.join(ROOT, "block_sparse_long_qk_amd", "csrc", name)
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def counter_traffic(kernel, workload):
    """Counter bytes per step (over all of the step's launches of the kernel)
    recorded for this kernel on this workload with its current sources, else
    None."""
    rec = COUNTER_TRAFFIC.get(kernel)
    if rec is None or COUNTER_WORKLOAD.get(kernel, "prefill_128k") != workload:
        return None
    nbytes, shas = rec
    if any(source_sha16(f) != s for f, s in shas.items()):
        return None
    return nbytes


def algorithmic_work(w):
    """Algorithmic work of one call on workload w: FLOPs of the index scoring,
    of the attention (and its local-block and non-local parts), the bytes of
    the top-k stage, the non-local (row, block) edges of the attention, and the
    per-row token counts."""
    import numpy as np
    pos = w.offset + np.arange(w.n_q, dtype=np.int64)
    local = pos // w.block_size
    f_idx = 2.0 * w.index_dim * w.h_kv * w.batch * float(np.sum(pos + 1))
    many = local + 1 > w.topk
    t_size = np.where(many, (w.topk - 1) * w.block_size + pos % w.block_size + 1, pos + 1)
    f_attn = 4.0 * w.head_dim * w.h_q * w.batch * float(np.sum(t_size))
    f_local = 4.0 * w.head_dim * w.h_q * w.batch * float(np.sum(pos % w.block_size + 1))
    topk_bytes = 4.0 * w.h_kv * w.batch * float(np.sum(local + 1)) + 4.0 * w.topk * w.h_kv * w.batch * w.n_q
    edges = float(np.sum(np.minimum(local, w.topk - 1))) * w.h_kv * w.batch
    return {"f_idx": f_idx, "f_attn": f_attn, "f_local": f_local, "f_nonlocal": f_attn - f_local,
            "topk_bytes": topk_bytes, "edges": edges, "t_size": t_size}


def decode_bytes(w):
    """HBM bytes one decode step must move: every index key once, the K/V of the
    selected tokens, Q, index-q, the output and the block indices."""
    t_size = algorithmic_work(w)["t_size"]
    eb = 1.0 if w.index_dtype == "fp8" else 2.0   # bytes per index element
    ekv = 1.0 if w.kv_dtype == "fp8" else 2.0     # bytes per K/V element
    ik = eb * w.batch * w.n_kv * w.index_dim
    kv = ekv * 2 * w.head_dim * w.h_kv * w.batch * float(t_size.sum())
    small = (2.0 * w.batch * w.n_q * 2 * w.h_q * w.head_dim + eb * w.batch * w.n_q * w.h_kv * w.index_dim
             + 4.0 * w.batch * w.h_kv * w.topk)
    return ik + kv + small


def kernel_work(name, w, wk):
    """(bound, algorithmic work per launch, unit) of one kernel of the step.
    Scoring and attention are MFMA-bound by the method (their FLOPs); the
    top-k is HBM-bound (its bytes).  The attention kernels also get the bytes
    their KV-outer design moves per (row, block) edge: the gathered query
    rows (2 B x G x d) and the partial (12-bit codes, 1.5 B x G x d) with its
    exponents (4 B per head) and log-sum-exps (4 B per head), written by the
    tiles and read by the merge."""
    G = w.h_q // w.h_kv
    edge_q = 2.0 * G * w.head_dim
    edge_part = 1.5 * G * w.head_dim + 4.0 * G + 4.0 * G
    if name.startswith("k_index_scores"):
        return "mfma", wk["f_idx"], "flop", None
    if name == "k_index_small":   # decode: a stream over every index key
        return "hbm", (1.0 if w.index_dtype == "fp8" else 2.0) * w.batch * w.n_kv * w.index_dim, "byte", None
    if name == "k_attn_rows":     # decode: the selected tokens' K and V
        ekv = 1.0 if w.kv_dtype == "fp8" else 2.0
        return "hbm", ekv * 2 * w.head_dim * w.h_kv * w.batch * float(wk["t_size"].sum()), "byte", None
    if name == "k_block_topk":
        return "hbm", wk["topk_bytes"], "byte", None
    if name == "k_attn_tiles":
        return "mfma", wk["f_nonlocal"], "flop", wk["edges"] * (edge_q + edge_part)
    if name == "k_attn_local_merge":
        rows = float(w.batch * w.n_q)
        local_bytes = rows * w.h_q * w.head_dim * 2.0 * 2 + rows * w.h_q * 4.0   # q and out, lse
        return "mfma", wk["f_local"], "flop", wk["edges"] * edge_part + local_bytes
    return None, None, None, None


def timed_steps(call, steps, warmup, stream, marked=None):
    """Warm up, then time exactly `steps` calls bracketed by synchronisations.
    With `marked` (a function of (events) that runs one marked call and
    returns its marks), the timed calls are marked ones: per-kernel times and
    per-step times are read from their events."""
    import torch
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    sets = []
    if marked is not None:
        for _ in range(steps):
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(MAX_MARKS)]
            for e in evs:
                e.record(stream)   # creates the underlying events
            sets.append(evs)
        torch.cuda.synchronize()
    marks = []
    w0 = time.perf_counter()
    a.record(stream)
    for s in range(steps):
        if marked is not None:
            marks.append(marked(sets[s]))
        else:
            call()
    b.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - w0) * 1e3 / steps
    ms = a.elapsed_time(b) / steps
    res = {"ms": ms, "wall_ms": wall}
    if marks:
        per_step = [m[0][1].elapsed_time(m[-1][2]) for m in marks]
        kern = {}
        for m in marks:
            seen = {}
            for name, e0, e1 in m:
                seen.setdefault(name, []).append(e0.elapsed_time(e1))
            for name, ts in seen.items():
                d = kern.setdefault(name, {"launches_per_step": len(ts), "ms": []})
                d["ms"].extend(ts)
        res["per_step"] = per_step
        res["kernels"] = {n: {"launches_per_step": d["launches_per_step"], "avg_ms": sum(d["ms"]) / len(d["ms"])}
                          for n, d in kern.items()}
    return res


def stats(xs):
    import numpy as np
    x = np.asarray(xs, dtype=np.float64)
    return {"median": round(float(np.median(x)), 4), "min": round(float(x.min()), 4),
            "p90": round(float(np.percentile(x, 90)), 4), "mean": round(float(x.mean()), 4), "n": int(len(x))}


def problem_of(w):
    import block_sparse_long_qk_amd as msa
    return msa.Problem.make(w.batch, w.n_q, w.n_kv, w.h_q, w.h_kv, w.head_dim, w.index_dim, w.block_size, w.topk,
                            w.q_offset, w.scale,
                            index_dtype=msa.DTYPE_FP8_E4M3 if w.index_dtype == "fp8" else msa.DTYPE_BF16,
                            kv_dtype=msa.DTYPE_FP8_E4M3 if w.kv_dtype == "fp8" else msa.DTYPE_BF16)


def kernel_table(w, kernels, ms_step):
    """Per kernel of a step: time, share of the step, algorithmic work and its
    fraction of the roofline (and, for the attention kernels, the rate of the
    bytes their design moves)."""
    wk = algorithmic_work(w)
    out = {}
    for name, d in sorted(kernels.items(), key=lambda kv: -kv[1]["avg_ms"] * kv[1]["launches_per_step"]):
        ms = d["avg_ms"]
        e = {"avg_ms": round(ms, 4), "launches_per_step": d["launches_per_step"],
             "share_of_step": round(ms * d["launches_per_step"] / ms_step, 4)}
        bound, work, unit, design_bytes = kernel_work(name, w, wk)
        # the step's work of this kernel over its time summed over the step's
        # launches (the overlapped passes launch each attention and scoring
        # kernel once per pass)
        tot = ms * d["launches_per_step"]
        if bound == "mfma":
            e["tflops"] = round(work / (tot * 1e-3) / 1e12, 1)
            e["frac_mfma"] = round(work / (tot * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
        elif bound == "hbm":
            e["gbs"] = round(work / (tot * 1e-3) / 1e9, 1)
            e["frac_hbm"] = round(work / (tot * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
        if design_bytes is not None:
            e["design_gbs"] = round(design_bytes / (tot * 1e-3) / 1e9, 1)
            e["design_frac_hbm"] = round(design_bytes / (tot * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
        traffic = counter_traffic(name, w.name)
        if traffic is not None:
            e["counter_bytes"] = traffic
            e["counter_frac_hbm"] = round(traffic / (tot * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
        out[name] = e
    return out


def roofline_of(w, kernels):
    """The roofline object of the step's dominant kernel (the largest total
    time per step)."""
    wk = algorithmic_work(w)
    name, d = max(kernels.items(), key=lambda kv: kv[1]["avg_ms"] * kv[1]["launches_per_step"])
    bound, work, unit, _ = kernel_work(name, w, wk)
    ms, n = d["avg_ms"], d["launches_per_step"]
    work /= n  # per launch: the step's work spread over its launches
    if bound == "mfma":
        ach, peak, u = work / (ms * 1e-3) / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"
    else:
        ach, peak, u = work / (ms * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s"
    traffic = counter_traffic(name, w.name)
    return {"bound": bound, "kernel": name, "achieved": round(ach, 2), "peak": peak, "unit": u,
            "frac": round(ach / peak, 4), "traffic": None if traffic is None else traffic / n, "avg_ms": round(ms, 4),
            "launches_per_step": n}


def gpu_leg(w, steps, warmup, stream, paged=False, kl=False, stages=True, check=False):
    import torch
    import block_sparse_long_qk_amd as msa
    import synth
    print(f"[bench] generating {w.name} inputs", file=sys.stderr, flush=True)
    x = synth.device_inputs(w)
    p = problem_of(w)
    f = msa.alloc_outputs(p)
    sp = stream.cuda_stream

    def step():
        msa.forward(p, x["q"], x["k"], x["v"], x["iq"], x["ik"], f["out"], f["block_idx"], f["lse"], f["workspace"],
                    stream=sp)

    def marked(evs):
        return msa.forward_marked(p, x["q"], x["k"], x["v"], x["iq"], x["ik"], f["out"], f["block_idx"], f["lse"],
                                  f["workspace"], evs, stream=sp)

    print(f"[bench] timing {steps} steps of {w.name}", file=sys.stderr, flush=True)
    # prefill: the timed steps themselves are marked (an event per kernel, a
    # few microseconds in a step of tens of milliseconds); decode: plain steps
    # for the rate, then as many marked steps for the per-kernel times
    if w.n_q > 1:
        t = timed_steps(step, steps, warmup, stream, marked=marked)
    else:
        t = timed_steps(step, steps, warmup, stream)
        tm = timed_steps(step, steps, 0, stream, marked=marked)
        t["per_step"], t["kernels"] = tm["per_step"], tm["kernels"]
    res = {"ms_step": t["ms"], "wall_ms_step": t["wall_ms"], "per_step": t["per_step"], "kernels": t["kernels"]}

    if check:
        # the timed call's block indices against the staged calls' (index scores,
        # then top-k on the pooled tensor): the fused launch and the two stages
        # must agree bit for bit
        fused = f["block_idx"].clone()
        pooled = torch.empty((w.batch, w.h_kv, w.n_q, w.n_blk), dtype=torch.float32, device="cuda")
        staged = torch.empty_like(fused)
        msa.index_scores(p, x["iq"], x["ik"], pooled, sp)
        msa.block_topk(p, pooled, staged, sp)
        torch.cuda.synchronize()
        res["timed_equals_staged"] = bool(torch.equal(fused, staged))
        del pooled, staged, fused

    if w.n_q == 1:
        # decode: the same step captured once as a HIP graph and replayed (the
        # calls enqueue kernels only, so the step captures as it is)
        def step_cur():  # on the current stream, which is the capture stream while capturing
            msa.forward(p, x["q"], x["k"], x["v"], x["iq"], x["ik"], f["out"], f["block_idx"], f["lse"],
                        f["workspace"])

        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step_cur()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step_cur()
        res["ms_step_graph"] = timed_steps(graph.replay, steps, warmup, stream)["ms"]
        del graph

    if stages:
        # each entry point alone, same stream, its own buffers
        pooled = torch.empty((w.batch, w.h_kv, w.n_q, w.n_blk), dtype=torch.float32, device="cuda")
        bidx = torch.empty_like(f["block_idx"])
        attn_ws = torch.empty(max(msa.workspace_size(p, msa.OP_SPARSE_ATTN), 256), dtype=torch.uint8, device="cuda")
        res["ms_index"] = timed_steps(lambda: msa.index_scores(p, x["iq"], x["ik"], pooled, sp), steps, 1, stream)["ms"]
        res["ms_topk"] = timed_steps(lambda: msa.block_topk(p, pooled, bidx, sp), steps, 1, stream)["ms"]
        res["ms_attn"] = timed_steps(lambda: msa.sparse_attn_fwd(p, x["q"], x["k"], x["v"], bidx, f["out"], f["lse"],
                                                                 attn_ws, stream=sp), steps, 1, stream)["ms"]
        del pooled, bidx, attn_ws
    if kl and msa.workspace_size(p, msa.OP_INDEX_KL) > 0:
        # the KL alignment pass on this step's selection and lse
        kl_out = torch.empty((w.batch, w.h_kv, w.n_q), dtype=torch.float32, device="cuda")
        kl_ws = torch.empty(max(msa.workspace_size(p, msa.OP_INDEX_KL), 256), dtype=torch.uint8, device="cuda")
        lse_index = torch.empty_like(kl_out)
        run_kl = lambda: msa.index_kl(p, x["q"], x["k"], x["iq"], x["ik"], f["block_idx"], f["lse"], kl_out, kl_ws,
                                      stream=sp, lse_index=lse_index)
        res["ms_kl"] = timed_steps(run_kl, steps, warmup, stream)["ms"]
        res["kl_mean"] = float(kl_out.mean().item())
        # its gradient into the index projections (teacher detached)
        d_iq, d_ik = torch.empty_like(x["iq"]), torch.empty_like(x["ik"])
        kb_ws = torch.empty(msa.workspace_size(p, msa.OP_INDEX_KL_BWD), dtype=torch.uint8, device="cuda")
        run_klb = lambda: msa.index_kl_bwd(p, x["q"], x["k"], x["iq"], x["ik"], f["block_idx"], f["lse"], lse_index,
                                           d_iq, d_ik, workspace=kb_ws, stream=sp)
        res["ms_kl_bwd"] = timed_steps(run_klb, steps, warmup, stream)["ms"]
        # the pair that keeps the teacher: the KL pass storing it (fp16 per
        # (row, slot, key)), and the backward reading it instead of forming S
        teacher = torch.empty(msa.teacher_shape(p), dtype=torch.float16, device="cuda")
        run_klt = lambda: msa.index_kl_teacher(p, x["q"], x["k"], x["iq"], x["ik"], f["block_idx"], f["lse"], kl_out,
                                               lse_index, teacher, kl_ws, stream=sp)
        res["ms_kl_teacher"] = timed_steps(run_klt, steps, warmup, stream)["ms"]
        run_klbt = lambda: msa.index_kl_bwd_teacher(p, x["iq"], x["ik"], f["block_idx"], teacher, lse_index, d_iq,
                                                    d_ik, workspace=kb_ws, stream=sp)
        res["ms_kl_bwd_teacher"] = timed_steps(run_klbt, steps, warmup, stream)["ms"]
        del d_iq, d_ik, kb_ws, lse_index, teacher
        # dense mode (the indexer warmup): dense attention, then the KL over every visible token
        d_out = torch.empty_like(f["out"])
        d_lse = torch.empty_like(f["lse"])
        run_dense = lambda: msa.dense_attn_fwd(p, x["q"], x["k"], x["v"], d_out, d_lse, stream=sp)
        run_dkl = lambda: msa.dense_index_kl(p, x["q"], x["k"], x["iq"], x["ik"], d_lse, kl_out, stream=sp)
        res["ms_dense_attn"] = timed_steps(run_dense, max(1, steps // 2), 1, stream)["ms"]
        res["ms_dense_kl"] = timed_steps(run_dkl, max(1, steps // 2), 1, stream)["ms"]
        del kl_out, kl_ws, d_out, d_lse
        # the main-branch backward on this step's selection, out and lse
        dout = synth.device_dout(w)
        dq, dk, dv = torch.empty_like(x["q"]), torch.empty_like(x["k"]), torch.empty_like(x["v"])
        b_ws = torch.empty(max(msa.workspace_size(p, msa.OP_SPARSE_ATTN_BWD), 256), dtype=torch.uint8, device="cuda")
        run_bwd = lambda: msa.sparse_attn_bwd(p, x["q"], x["k"], x["v"], f["block_idx"], f["out"], f["lse"], dout, dq,
                                              dk, dv, b_ws, stream=sp)
        res["ms_bwd"] = timed_steps(run_bwd, steps, warmup, stream)["ms"]
        del dout, dq, dk, dv, b_ws
    if paged:
        # the same step through msa_forward_v, the caches re-laid as a shuffled page pool
        ref = {key: f[key].clone() for key in ("out", "block_idx", "lse")}
        vl, kp, vp, ikp = to_pages(w, x, seed=w.seed)
        print(f"[bench] timing {steps} paged steps of {w.name}", file=sys.stderr, flush=True)

        def paged_step():
            msa.forward(p, x["q"], kp, vp, x["iq"], ikp, f["out"], f["block_idx"], f["lse"], f["workspace"],
                        stream=sp, varlen=vl)

        res["ms_step_paged"] = timed_steps(paged_step, steps, warmup, stream)["ms"]
        res["paged_equal"] = (torch.equal(ref["block_idx"], f["block_idx"]) and torch.equal(ref["lse"], f["lse"])
                              and torch.equal(ref["out"].view(torch.int16), f["out"].view(torch.int16)))
        del ref, kp, vp, ikp, vl
    del x, f
    torch.cuda.empty_cache()
    return res


def cold_leg(w, runs, stream, scrub_bytes=512 << 20):
    """Warm and cold steps of a small workload: warm = back-to-back steps;
    cold = each step right after writing a scrub buffer larger than the
    Infinity Cache (256 MiB), so that the inputs start in HBM."""
    import torch
    import block_sparse_long_qk_amd as msa
    import synth
    x = synth.device_inputs(w)
    p = problem_of(w)
    f = msa.alloc_outputs(p)
    sp = stream.cuda_stream
    scrub = torch.empty(scrub_bytes, dtype=torch.uint8, device="cuda")

    def step():
        msa.forward(p, x["q"], x["k"], x["v"], x["iq"], x["ik"], f["out"], f["block_idx"], f["lse"], f["workspace"],
                    stream=sp)

    warm = []
    for _ in range(3):
        step()
    for _ in range(runs):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step()
        b.record(stream)
        b.synchronize()
        warm.append(a.elapsed_time(b))
    cold = []
    for r in range(runs):
        scrub.fill_(r & 255)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step()
        b.record(stream)
        b.synchronize()
        cold.append(a.elapsed_time(b))
    del x, f, scrub
    torch.cuda.empty_cache()
    return {"workload": w.name, "warm_ms": stats(warm), "cold_ms": stats(cold),
            "scrub": f"{scrub_bytes >> 20} MiB written before each cold step"}


def to_pages(w, x, seed):
    """Re-lay the contiguous caches of x as a page pool in the paged layout
    (k/v [pages][h_kv][Bk][d], index_k [pages][Bk][d_idx]) with a seeded random
    page permutation, and describe it with a Varlen of uniform lengths.  The
    contiguous k, v and index_k are released from x as they are copied."""
    import numpy as np
    import torch
    import block_sparse_long_qk_amd as msa
    B, hk, bk, d, di, pps = w.batch, w.h_kv, w.block_size, w.head_dim, w.index_dim, w.n_blk
    assert w.n_kv == pps * bk, "the paged bench leg takes whole blocks"
    dev = x["q"].device
    perm = torch.from_numpy(np.random.default_rng(seed).permutation(B * pps)).to(dev)
    pool = {}
    for name, page_shape in (("k", (hk, bk, d)), ("v", (hk, bk, d)), ("ik", (bk, di))):
        dst = torch.empty((B * pps,) + page_shape, dtype=torch.bfloat16, device=dev)
        for b in range(B):
            src = x[name][b].view(hk, pps, bk, d).transpose(0, 1) if name != "ik" else x[name][b].view(pps, bk, di)
            dst.index_copy_(0, perm[b * pps:(b + 1) * pps], src)
        x[name] = None
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        pool[name] = dst
    i32 = lambda a: a.to(torch.int32).contiguous()
    vl = msa.Varlen.make(qo_lens=i32(torch.full((B,), w.n_q, device=dev)),
                         kv_lens=i32(torch.full((B,), w.n_kv, device=dev)),
                         q_starts=i32(torch.arange(B, device=dev) * w.n_q), total_q=B * w.n_q,
                         page_table=i32(perm.view(B, pps)), num_pages=B * pps)
    return vl, pool["k"], pool["v"], pool["ik"]


def cpu_leg(w, n_positions, seed=0):
    """The oracle, as it stands, on a stratified sample of query positions of
    the same workload (all groups and heads; every position when n_positions
    >= n_q); input generation is not timed.  Returns the measured rate and the
    full-run time extrapolated from it: the pooling part scales with the sum
    of (p + 1) over positions, the attention part with the sum of |T|."""
    import numpy as np
    import oracle
    import synth
    rng = np.random.default_rng(seed)
    if n_positions >= w.n_q:
        rows = np.arange(w.n_q, dtype=np.int64)
    else:
        edges = np.linspace(0, w.n_q, n_positions + 1).astype(np.int64)
        rows = np.array([rng.integers(a, max(a + 1, z)) for a, z in zip(edges[:-1], edges[1:])], dtype=np.int64)
    plant = synth.plant_spec(w)
    t_pool = t_attn = 0.0
    for b in range(w.batch if w.n_q == 1 else 1):
        for g in range(w.h_kv):
            x = oracle.inputs_for_rows(w, b, g, rows, plant)
            t0 = time.perf_counter()
            pooled = oracle.pool(x["iq"], x["pos"], x["ik"], w.block_size)
            sel = oracle.select(pooled, x["pos"], w.block_size, w.topk)
            t_pool += time.perf_counter() - t0
            K, V = oracle.kv_for_blocks(w, b, g, sel)
            t0 = time.perf_counter()
            oracle.attend(x["q"], x["pos"], sel, K, V, w.block_size, w.scale)
            t_attn += time.perf_counter() - t0
    n_tok = len(rows) * (w.batch if w.n_q == 1 else 1)
    spent = t_pool + t_attn
    t_size = algorithmic_work(w)["t_size"]
    pos = w.offset + np.arange(w.n_q, dtype=np.int64)
    full = (t_pool * float(np.sum(pos + 1)) / float(np.sum(pos[rows] + 1))
            + t_attn * float(np.sum(t_size)) / float(np.sum(t_size[rows])))
    return {"rate": n_tok / spent, "spent": spent, "n_tok": n_tok, "full_s": full * (w.batch if w.n_q == 1 else 1)}


def host_description():
    """CPU model, logical CPUs, NUMA nodes of the host running the oracle."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        numa = len([n for n in os.listdir("/sys/devices/system/node") if n.startswith("node") and n[4:].isdigit()])
    except OSError:
        numa = None
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count()
    return {"cpu_model": model, "logical_cpus": os.cpu_count(), "cpus_available": affinity, "numa_nodes": numa}


def single_thread_c1():
    """The oracle on the whole 4K workload with one thread, in a child process
    (OpenMP fixes its thread count at start-up); the child never touches the GPU."""
    env = dict(os.environ, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, os.path.abspath(__file__), "--_cpu-c1"], env=env, capture_output=True,
                       text=True, timeout=600)
    if r.returncode != 0:
        return {"error": r.stderr[-300:]}
    return json.loads(r.stdout.strip().splitlines()[-1])


def line_for(w, g):
    """Rates and fractions of one prefill workload's marked steps."""
    wk = algorithmic_work(w)
    ms = g["ms_step"]
    kern = g["kernels"]
    t_attn = sum(d["avg_ms"] * d["launches_per_step"] for n, d in kern.items()
                 if n.startswith("k_attn") or n.startswith("k_plan") or n.startswith("k_scan"))
    t_idx = sum(d["avg_ms"] * d["launches_per_step"] for n, d in kern.items() if n.startswith("k_index_"))
    t_attn = max(t_attn, sum(d["avg_ms"] * d["launches_per_step"] for n, d in kern.items()
                             if n in ("k_attn_rows", "k_merge_rows")))
    frac = lambda f, t: round(f / (t * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4) if t > 0 else None
    t_topk = sum(d["avg_ms"] * d["launches_per_step"] for n, d in kern.items() if n == "k_block_topk")
    out = {"workload": w.name, "tokens_per_s": round(w.batch * w.n_q / (ms * 1e-3), 1), "ms_per_step": round(ms, 4),
           "step_ms": stats(g["per_step"]),
           "combined_mfma_frac": round((wk["f_idx"] + wk["f_attn"]) / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
           "scoring_ms": round(t_idx, 4),
           "scoring_frac_mfma": frac(wk["f_idx"], t_idx),
           "attention_ms": round(t_attn, 4),
           "attention_frac_mfma": frac(wk["f_attn"], t_attn),
           "kernels": kernel_table(w, kern, ms)}
    if t_topk > 0:
        out["topk_ms"] = round(t_topk, 4)
        out["topk_frac_hbm"] = round(wk["topk_bytes"] / (t_topk * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prefill_128k")
    ap.add_argument("--decode-workload", default="decode_256k")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the 32K, 1M-chunk and cold-cache lines")
    ap.add_argument("--cpu-positions", type=int, default=3072)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-paged", action="store_true", help="skip the paged-cache (msa_forward_v) legs")
    ap.add_argument("--no-fp8", action="store_true", help="skip the FP8 (E4M3) index-input and K/V legs")
    ap.add_argument("--no-kl", action="store_true", help="skip the KL pass, the backward passes and dense mode")
    ap.add_argument("--_cpu-c1", action="store_true", help=argparse.SUPPRESS)
    args = ap.parse_args()
    if args._cpu_c1:
        import synth
        r = cpu_leg(synth.WORKLOADS["prefill_4k"], 1 << 30)
        print(json.dumps({"workload": "prefill_4k", "threads": int(os.environ.get("OMP_NUM_THREADS", "0") or 0),
                          "seconds": round(r["spent"], 3), "tokens_per_s": round(r["rate"], 2)}))
        return
    if args.gpus != 1:
        print("bench.py: this build runs on one GPU only; the multi-GPU sharding is a design note, "
              "not an implemented path (use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    torch.cuda.init()
    stream = torch.cuda.current_stream()
    # copy probe: 1 GiB device-to-device copy of known size, so that HBM byte
    # counters (FETCH_SIZE, WRITE_SIZE) can be scaled against a known transfer
    probe_src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
    probe_dst = torch.empty_like(probe_src)
    probe_dst.copy_(probe_src)
    torch.cuda.synchronize()
    # the same copy timed: the practical HBM rate of a plain stream (read + write),
    # reported beside the 8 TB/s spec as context for the HBM-bound stages
    copy_ms = timed_steps(lambda: probe_dst.copy_(probe_src), 5, 0, stream)["ms"]
    copy_gbs = 2.0 * (1 << 30) / (copy_ms * 1e-3) / 1e9
    del probe_src, probe_dst
    w = synth.WORKLOADS[args.workload]
    g = gpu_leg(w, args.steps, args.warmup, stream, paged=not args.no_paged, kl=not args.no_kl, check=True)
    wk = algorithmic_work(w)
    ms = g["ms_step"]
    tok_s = w.batch * w.n_q / (ms * 1e-3)
    stages = {
        "index_scores": {"ms": round(g["ms_index"], 4),
                         "frac_mfma": round(wk["f_idx"] / (g["ms_index"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)},
        "block_topk": {"ms": round(g["ms_topk"], 4),
                       "gbs": round(wk["topk_bytes"] / (g["ms_topk"] * 1e-3) / 1e9, 1),
                       "frac_hbm": round(wk["topk_bytes"] / (g["ms_topk"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
        "sparse_attn": {"ms": round(g["ms_attn"], 4),
                        "frac_mfma": round(wk["f_attn"] / (g["ms_attn"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)},
    }
    main_line = line_for(w, g)
    line = {
        "metric": "MSA prefill tokens/s @128K; decode tokens/s @256K KV; % of roofline",
        "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "n_q": w.n_q, "n_kv": w.n_kv, "h_q": w.h_q, "h_kv": w.h_kv,
                   "head_dim": w.head_dim, "index_dim": w.index_dim, "block_size": w.block_size, "topk": w.topk},
        "roofline": roofline_of(w, g["kernels"]),
        "step_ms": main_line["step_ms"],
        "combined_mfma_frac": main_line["combined_mfma_frac"],
        "scoring_frac_mfma": main_line["scoring_frac_mfma"],
        "attention_frac_mfma": main_line["attention_frac_mfma"],
        "kernels": main_line["kernels"],
        "timed_equals_staged": g["timed_equals_staged"],
        "hbm_copy_gbs": round(copy_gbs, 1),
        "algorithmic_tflop_per_step": round((wk["f_idx"] + wk["f_attn"]) / 1e12, 3),
        "stages_alone": stages,
        "wall_ms_per_step": round(g["wall_ms_step"], 4),
    }

    if not args.no_decode:
        wd = synth.WORKLOADS[args.decode_workload]
        gd = gpu_leg(wd, args.steps, args.warmup, stream, paged=not args.no_paged)
        db = decode_bytes(wd)
        kd = {n: {"avg_ms": round(d["avg_ms"], 4)} for n, d in gd["kernels"].items()}
        if "k_index_small" in gd["kernels"]:
            t = gd["kernels"]["k_index_small"]["avg_ms"]
            ikb = (1.0 if wd.index_dtype == "fp8" else 2.0) * wd.batch * wd.n_kv * wd.index_dim
            kd["k_index_small"]["gbs"] = round(ikb / (t * 1e-3) / 1e9, 1)
            kd["k_index_small"]["frac_hbm"] = round(ikb / (t * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
        line["decode"] = {
            "workload": wd.name, "tokens_per_s": round(wd.batch / (gd["ms_step"] * 1e-3), 1),
            "ms_per_step": round(gd["ms_step"], 4), "step_ms_marked": stats(gd["per_step"]),
            "bytes_per_step": db,
            "hbm_gbs": round(db / (gd["ms_step"] * 1e-3) / 1e9, 1),
            "frac_hbm": round(db / (gd["ms_step"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "frac_of_copy": round(db / (gd["ms_step"] * 1e-3) / 1e9 / copy_gbs, 4),
            "kernels": kd,
            "stages_alone_ms": {"index_scores": round(gd["ms_index"], 4), "block_topk": round(gd["ms_topk"], 4),
                                "sparse_attn": round(gd["ms_attn"], 4)},
            "graph_ms_per_step": round(gd["ms_step_graph"], 4),
            "graph_tokens_per_s": round(wd.batch / (gd["ms_step_graph"] * 1e-3), 1),
        }

    if not args.no_extra:
        # the other prefill configurations as lines of their own
        for name in ("prefill_32k", "chunked_1m"):
            we = synth.WORKLOADS[name]
            ge = gpu_leg(we, args.steps, args.warmup, stream, stages=False)
            line[name] = line_for(we, ge)
        line["cold_cache"] = [cold_leg(synth.WORKLOADS[n], max(5, args.steps // 2), stream)
                              for n in ("prefill_4k", "prefill_32k")]

    if "ms_kl" in g:
        t_size = wk["t_size"]
        # S = Q K^T for every head and Z = IQ IK^T for every group, over each row's tokens
        f_kl = 2.0 * (w.head_dim * w.h_q + w.index_dim * w.h_kv) * w.batch * float(t_size.sum())
        line["kl"] = {"ms": round(g["ms_kl"], 4), "tflops": round(f_kl / (g["ms_kl"] * 1e-3) / 1e12, 1),
                      "frac_mfma": round(f_kl / (g["ms_kl"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                      "mean_kl": round(g["kl_mean"], 5)}
        # its gradient: S for every head, then Z, d_index_k and d_index_q for every group
        f_klb = 2.0 * (w.head_dim * w.h_q + 3 * w.index_dim * w.h_kv) * w.batch * float(t_size.sum())
        line["kl_backward"] = {"ms": round(g["ms_kl_bwd"], 4),
                               "tflops": round(f_klb / (g["ms_kl_bwd"] * 1e-3) / 1e12, 1),
                               "frac_mfma": round(f_klb / (g["ms_kl_bwd"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        # with the teacher stored: the KL pass also writes it (2 bytes per (row, slot, key));
        # the backward reads it (no S), then Z, d_index_k and d_index_q for every group
        t_bytes = 2.0 * w.batch * w.h_kv * w.n_q * (w.topk + 1) * w.block_size
        f_klbt = 2.0 * 3 * w.index_dim * w.h_kv * w.batch * float(t_size.sum())
        line["kl_teacher"] = {"ms": round(g["ms_kl_teacher"], 4), "teacher_gb": round(t_bytes / 1e9, 2),
                              "kl_plus_bwd_ms": round(g["ms_kl_teacher"] + g["ms_kl_bwd_teacher"], 4)}
        line["kl_backward_teacher"] = {"ms": round(g["ms_kl_bwd_teacher"], 4),
                                       "tflops": round(f_klbt / (g["ms_kl_bwd_teacher"] * 1e-3) / 1e12, 1)}
        # dense mode: every visible token (sum over rows of p + 1)
        import numpy as np
        n_vis = float(np.sum(w.offset + np.arange(w.n_q, dtype=np.int64) + 1)) * w.batch
        f_dense = 4.0 * w.head_dim * w.h_q * n_vis
        f_dkl = 2.0 * (w.head_dim * w.h_q + w.index_dim * w.h_kv) * n_vis
        # backward: S recomputed, dP, dV, dK, dQ over each row's tokens (five products)
        f_bwd = 2.5 * wk["f_attn"]
        line["backward"] = {"ms": round(g["ms_bwd"], 4), "tflops": round(f_bwd / (g["ms_bwd"] * 1e-3) / 1e12, 1),
                            "frac_mfma": round(f_bwd / (g["ms_bwd"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        line["dense"] = {
            "attn_ms": round(g["ms_dense_attn"], 3),
            "attn_tflops": round(f_dense / (g["ms_dense_attn"] * 1e-3) / 1e12, 1),
            "attn_frac_mfma": round(f_dense / (g["ms_dense_attn"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "kl_ms": round(g["ms_dense_kl"], 3),
            "kl_tflops": round(f_dkl / (g["ms_dense_kl"] * 1e-3) / 1e12, 1),
            "kl_frac_mfma": round(f_dkl / (g["ms_dense_kl"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "msa_speedup_over_dense": round(g["ms_dense_attn"] / ms, 2)}

    if not args.no_paged:
        # the same steps with the caches in a shuffled page pool (msa_forward_v, uniform lengths)
        line["paged"] = {"prefill_ms_per_step": round(g["ms_step_paged"], 4),
                         "prefill_tokens_per_s": round(w.batch * w.n_q / (g["ms_step_paged"] * 1e-3), 1),
                         "prefill_vs_contiguous": round(ms / g["ms_step_paged"], 4),
                         "prefill_bitwise_equal": g["paged_equal"]}
        if not args.no_decode:
            line["paged"].update({
                "decode_ms_per_step": round(gd["ms_step_paged"], 4),
                "decode_tokens_per_s": round(wd.batch / (gd["ms_step_paged"] * 1e-3), 1),
                "decode_frac_hbm": round(db / (gd["ms_step_paged"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                "decode_vs_contiguous": round(gd["ms_step"] / gd["ms_step_paged"], 4),
                "decode_bitwise_equal": gd["paged_equal"]})

    if not args.no_fp8:
        # the same steps with E4M3 index inputs (the main branch stays bf16)
        wf = w.replace(name=w.name + "_fp8_index", index_dtype="fp8")
        gf = gpu_leg(wf, args.steps, args.warmup, stream)
        t8 = sum(d["avg_ms"] for n, d in gf["kernels"].items() if n.startswith("k_index_scores"))
        line["fp8_index"] = {"prefill_ms_per_step": round(gf["ms_step"], 4),
                             "prefill_tokens_per_s": round(w.batch * w.n_q / (gf["ms_step"] * 1e-3), 1),
                             "scoring_ms": round(t8, 4),
                             "scoring_frac_fp8_mfma": round(wk["f_idx"] / (t8 * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4),
                             "index_scores_alone_ms": round(gf["ms_index"], 4)}
        if not args.no_decode:
            wdf = wd.replace(name=wd.name + "_fp8_index", index_dtype="fp8")
            gdf = gpu_leg(wdf, args.steps, args.warmup, stream)
            dbf = decode_bytes(wdf)
            line["fp8_index"].update({
                "decode_ms_per_step": round(gdf["ms_step"], 4),
                "decode_tokens_per_s": round(wdf.batch / (gdf["ms_step"] * 1e-3), 1),
                "decode_bytes_per_step": dbf,
                "decode_frac_hbm": round(dbf / (gdf["ms_step"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                "decode_index_ms": round(gdf["kernels"].get("k_index_small", {"avg_ms": float("nan")})["avg_ms"], 4)})
        # E4M3 K/V caches (the index branch bf16), then both branches E4M3 for decode
        wk8 = w.replace(name=w.name + "_fp8_kv", kv_dtype="fp8")
        gk = gpu_leg(wk8, args.steps, args.warmup, stream)
        line["fp8_kv"] = {"prefill_ms_per_step": round(gk["ms_step"], 4),
                          "prefill_tokens_per_s": round(w.batch * w.n_q / (gk["ms_step"] * 1e-3), 1),
                          "sparse_attn_alone_ms": round(gk["ms_attn"], 4)}
        if not args.no_decode:
            for key, wdk in (("decode", wd.replace(name=wd.name + "_fp8_kv", kv_dtype="fp8")),
                             ("decode_fp8_both", wd.replace(name=wd.name + "_fp8_both", kv_dtype="fp8",
                                                            index_dtype="fp8"))):
                gdk = gpu_leg(wdk, args.steps, args.warmup, stream)
                dbk = decode_bytes(wdk)
                line["fp8_kv"].update({
                    key + "_ms_per_step": round(gdk["ms_step"], 4),
                    key + "_tokens_per_s": round(wdk.batch / (gdk["ms_step"] * 1e-3), 1),
                    key + "_bytes_per_step": dbk,
                    key + "_frac_hbm": round(dbk / (gdk["ms_step"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)})

    if not args.no_cpu_baseline:
        print("[bench] oracle CPU baseline", file=sys.stderr, flush=True)
        r = cpu_leg(w, args.cpu_positions)
        threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
        host = host_description()
        st = single_thread_c1()
        line["cpu_baseline"] = {
            "value": round(r["rate"], 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{r['n_tok']} query positions (stratified over the {w.n_q}-token prefill, all {w.h_kv} "
                      f"groups / {w.h_q} heads), {r['spent']:.1f} s of oracle time",
            "extrapolated_full_run_s": round(r["full_s"], 1),
            "extrapolated_note": "extrapolated, not measured: pooling time scaled by sum(p+1), attention by sum|T|",
            "host": host, "single_thread_prefill_4k": st}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
