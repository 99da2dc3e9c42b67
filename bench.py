"""Benchmark of the MSA forward pass on one MI355X.

One step = one msa_forward call (index scores + block max-pool, block top-k,
gather plan, sparse attention, merge) over the 128K-token causal prefill
(batch 1, 64 query heads on 8 KV heads, head dim 128, index dim 128, Bk 128,
k 16), inputs seeded and synthetic, resident in HBM before timing starts.
Prints one JSON line: prefill tokens/s (the value), the decode rate at a
256K-token cache (64 sequences), per-stage times, the roofline of the dominant
kernel, the same two steps with the caches in a shuffled page pool
(msa_forward_v), the same two steps with FP8 (E4M3) index inputs and with
FP8 K/V caches, the KL pass and both backward passes and dense mode at 128K,
and the oracle's CPU rate on a bounded sample of the same workload.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
# HBM bytes of one standalone k_index_scores<128, 0> launch at 128K, from
# rocprofv3 FETCH_SIZE (x2, calibrated on a 1 GiB copy) + WRITE_SIZE (x1); see
# profiles/prefill_128k_attention_index_counters.md.  Valid for this kernel
# version only: re-measure (or set None) when the kernel changes.
INDEX_TRAFFIC_BYTES = (2.5965e6 * 2 + 2.335e6) * 1024
# The same for one msa_sparse_attn_fwd at 128K: k_attn_tiles<false> plus
# k_attn_local_merge (the plan kernels add under 1%).
ATTN_TRAFFIC_BYTES = ((1.7700e7 + 1.8653e7) * 2 + 3.1715e7 + 2.2894e6) * 1024


def algorithmic_work(w):
    """Algorithmic FLOPs of the index scoring and of the attention, and the
    bytes of the top-k stage, for one call on workload w."""
    import numpy as np
    pos = w.offset + np.arange(w.n_q, dtype=np.int64)
    local = pos // w.block_size
    f_idx = 2.0 * w.index_dim * w.h_kv * w.batch * float(np.sum(pos + 1))
    many = local + 1 > w.topk
    t_size = np.where(many, (w.topk - 1) * w.block_size + pos % w.block_size + 1, pos + 1)
    f_attn = 4.0 * w.head_dim * w.h_q * w.batch * float(np.sum(t_size))
    topk_bytes = 4.0 * w.h_kv * w.batch * float(np.sum(local + 1)) + 4.0 * w.topk * w.h_kv * w.batch * w.n_q
    return f_idx, f_attn, topk_bytes, t_size


def decode_bytes(w):
    """HBM bytes one decode step must move: every index key once, the K/V of the
    selected tokens, Q, index-q, the output and the block indices."""
    _, _, _, t_size = algorithmic_work(w)
    eb = 1.0 if w.index_dtype == "fp8" else 2.0   # bytes per index element
    ekv = 1.0 if w.kv_dtype == "fp8" else 2.0     # bytes per K/V element
    ik = eb * w.batch * w.n_kv * w.index_dim
    kv = ekv * 2 * w.head_dim * w.h_kv * w.batch * float(t_size.sum())
    small = (2.0 * w.batch * w.n_q * 2 * w.h_q * w.head_dim + eb * w.batch * w.n_q * w.h_kv * w.index_dim
             + 4.0 * w.batch * w.h_kv * w.topk)
    return ik + kv + small


class Timer:
    """HIP-event timing of repeated launches on one stream."""

    def __init__(self, stream):
        import torch
        self.stream = stream
        self.a = torch.cuda.Event(enable_timing=True)
        self.b = torch.cuda.Event(enable_timing=True)

    def run(self, fn, n):
        import torch
        torch.cuda.synchronize()
        self.a.record(self.stream)
        for _ in range(n):
            fn()
        self.b.record(self.stream)
        torch.cuda.synchronize()
        return self.a.elapsed_time(self.b) / n


def gpu_leg(w, steps, warmup, stream, paged=False, kl=False):
    import torch
    import block_sparse_long_qk_amd as msa
    import synth
    print(f"[bench] generating {w.name} inputs", file=sys.stderr, flush=True)
    x = synth.device_inputs(w)
    p = msa.Problem.make(w.batch, w.n_q, w.n_kv, w.h_q, w.h_kv, w.head_dim, w.index_dim, w.block_size, w.topk,
                         w.q_offset, w.scale,
                         index_dtype=msa.DTYPE_FP8_E4M3 if w.index_dtype == "fp8" else msa.DTYPE_BF16,
                         kv_dtype=msa.DTYPE_FP8_E4M3 if w.kv_dtype == "fp8" else msa.DTYPE_BF16)
    f = msa.alloc_outputs(p)
    sp = stream.cuda_stream

    def step():
        msa.forward(p, x["q"], x["k"], x["v"], x["iq"], x["ik"], f["out"], f["block_idx"], f["lse"], f["workspace"],
                    stream=sp)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] timing {steps} steps of {w.name}", file=sys.stderr, flush=True)
    t = Timer(stream)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ms_step = t.run(step, steps)
    wall = (time.perf_counter() - w0) * 1e3 / steps

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
        for _ in range(warmup):
            graph.replay()
        ms_graph = t.run(graph.replay, steps)
        del graph
    else:
        ms_graph = None

    # stages alone, same stream, same buffers
    pooled = f["workspace"][:4 * w.batch * w.h_kv * w.n_q * w.n_blk].view(torch.float32)
    pooled = pooled.view(w.batch, w.h_kv, w.n_q, w.n_blk)
    attn_ws = torch.empty(max(msa.workspace_size(p, msa.OP_SPARSE_ATTN), 256), dtype=torch.uint8, device="cuda")
    ms_idx = t.run(lambda: msa.index_scores(p, x["iq"], x["ik"], pooled, sp), steps)
    ms_topk = t.run(lambda: msa.block_topk(p, pooled, f["block_idx"], sp), steps)
    ms_attn = t.run(lambda: msa.sparse_attn_fwd(p, x["q"], x["k"], x["v"], f["block_idx"], f["out"], f["lse"],
                                                attn_ws, stream=sp), steps)
    res = {"ms_step": ms_step, "wall_ms_step": wall, "ms_index": ms_idx, "ms_topk": ms_topk, "ms_attn": ms_attn,
           "ms_step_graph": ms_graph}
    del attn_ws
    if kl and msa.workspace_size(p, msa.OP_INDEX_KL) > 0:
        # the KL alignment pass on this step's selection and lse
        kl_out = torch.empty((w.batch, w.h_kv, w.n_q), dtype=torch.float32, device="cuda")
        kl_ws = torch.empty(max(msa.workspace_size(p, msa.OP_INDEX_KL), 256), dtype=torch.uint8, device="cuda")
        lse_index = torch.empty_like(kl_out)
        run_kl = lambda: msa.index_kl(p, x["q"], x["k"], x["iq"], x["ik"], f["block_idx"], f["lse"], kl_out, kl_ws,
                                      stream=sp, lse_index=lse_index)
        for _ in range(warmup):
            run_kl()
        res["ms_kl"] = t.run(run_kl, steps)
        res["kl_mean"] = float(kl_out.mean().item())
        # its gradient into the index projections (teacher detached)
        d_iq, d_ik = torch.empty_like(x["iq"]), torch.empty_like(x["ik"])
        kb_ws = torch.empty(msa.workspace_size(p, msa.OP_INDEX_KL_BWD), dtype=torch.uint8, device="cuda")
        run_klb = lambda: msa.index_kl_bwd(p, x["q"], x["k"], x["iq"], x["ik"], f["block_idx"], f["lse"], lse_index,
                                           d_iq, d_ik, workspace=kb_ws, stream=sp)
        for _ in range(warmup):
            run_klb()
        res["ms_kl_bwd"] = t.run(run_klb, steps)
        del d_iq, d_ik, kb_ws, lse_index
        # dense mode (the indexer warmup): dense attention, then the KL over every visible token
        d_out = torch.empty_like(f["out"])
        d_lse = torch.empty_like(f["lse"])
        run_dense = lambda: msa.dense_attn_fwd(p, x["q"], x["k"], x["v"], d_out, d_lse, stream=sp)
        run_dkl = lambda: msa.dense_index_kl(p, x["q"], x["k"], x["iq"], x["ik"], d_lse, kl_out, stream=sp)
        run_dense()
        run_dkl()
        res["ms_dense_attn"] = t.run(run_dense, max(1, steps // 2))
        res["ms_dense_kl"] = t.run(run_dkl, max(1, steps // 2))
        del kl_out, kl_ws, d_out, d_lse
        # the main-branch backward on this step's selection, out and lse
        dout = synth.device_dout(w)
        dq, dk, dv = torch.empty_like(x["q"]), torch.empty_like(x["k"]), torch.empty_like(x["v"])
        b_ws = torch.empty(max(msa.workspace_size(p, msa.OP_SPARSE_ATTN_BWD), 256), dtype=torch.uint8, device="cuda")
        run_bwd = lambda: msa.sparse_attn_bwd(p, x["q"], x["k"], x["v"], f["block_idx"], f["out"], f["lse"], dout, dq,
                                              dk, dv, b_ws, stream=sp)
        for _ in range(warmup):
            run_bwd()
        res["ms_bwd"] = t.run(run_bwd, steps)
        del dout, dq, dk, dv, b_ws
    if paged:
        # the same step through msa_forward_v, the caches re-laid as a shuffled page pool
        ref = {key: f[key].clone() for key in ("out", "block_idx", "lse")}
        vl, kp, vp, ikp = to_pages(w, x, seed=w.seed)
        print(f"[bench] timing {steps} paged steps of {w.name}", file=sys.stderr, flush=True)

        def paged_step():
            msa.forward(p, x["q"], kp, vp, x["iq"], ikp, f["out"], f["block_idx"], f["lse"], f["workspace"],
                        stream=sp, varlen=vl)

        for _ in range(warmup):
            paged_step()
        res["ms_step_paged"] = t.run(paged_step, steps)
        res["paged_equal"] = (torch.equal(ref["block_idx"], f["block_idx"]) and torch.equal(ref["lse"], f["lse"])
                              and torch.equal(ref["out"].view(torch.int16), f["out"].view(torch.int16)))
        del ref, kp, vp, ikp, vl
    del x, f
    torch.cuda.empty_cache()
    return res


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
    the same workload (all groups and heads); input generation is not timed."""
    import numpy as np
    import oracle
    import synth
    rng = np.random.default_rng(seed)
    edges = np.linspace(0, w.n_q, n_positions + 1).astype(np.int64)
    rows = np.array([rng.integers(a, max(a + 1, z)) for a, z in zip(edges[:-1], edges[1:])], dtype=np.int64)
    plant = synth.plant_spec(w)
    spent = 0.0
    for b in range(w.batch if w.n_q == 1 else 1):
        for g in range(w.h_kv):
            x = oracle.inputs_for_rows(w, b, g, rows, plant)
            t0 = time.perf_counter()
            pooled = oracle.pool(x["iq"], x["pos"], x["ik"], w.block_size)
            sel = oracle.select(pooled, x["pos"], w.block_size, w.topk)
            spent += time.perf_counter() - t0
            K, V = oracle.kv_for_blocks(w, b, g, sel)
            t0 = time.perf_counter()
            oracle.attend(x["q"], x["pos"], sel, K, V, w.block_size, w.scale)
            spent += time.perf_counter() - t0
    n_tok = len(rows) * (w.batch if w.n_q == 1 else 1)
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return n_tok / spent, spent, n_tok, threads


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prefill_128k")
    ap.add_argument("--decode-workload", default="decode_256k")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--cpu-positions", type=int, default=3072)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-paged", action="store_true", help="skip the paged-cache (msa_forward_v) legs")
    ap.add_argument("--no-fp8", action="store_true", help="skip the FP8 (E4M3) index-input and K/V legs")
    ap.add_argument("--no-kl", action="store_true", help="skip the KL alignment pass")
    args = ap.parse_args()
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
    copy_ms = Timer(stream).run(lambda: probe_dst.copy_(probe_src), 5)
    copy_gbs = 2.0 * (1 << 30) / (copy_ms * 1e-3) / 1e9
    del probe_src, probe_dst
    w = synth.WORKLOADS[args.workload]
    g = gpu_leg(w, args.steps, args.warmup, stream, paged=not args.no_paged, kl=not args.no_kl)
    f_idx, f_attn, topk_bytes, _ = algorithmic_work(w)
    tok_s = w.batch * w.n_q / (g["ms_step"] * 1e-3)

    # dominant kernel of the step: the index-scoring GEMM (one launch per msa_index_scores call)
    idx_tflops = f_idx / (g["ms_index"] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": "k_index_scores", "achieved": round(idx_tflops, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(idx_tflops / PEAK_BF16_TFLOPS, 4),
                "traffic": INDEX_TRAFFIC_BYTES if (w.name == "prefill_128k" and INDEX_TRAFFIC_BYTES) else None}
    stages = {
        "index_scores": {"ms": round(g["ms_index"], 4), "tflops": round(idx_tflops, 1),
                         "frac_mfma": round(idx_tflops / PEAK_BF16_TFLOPS, 4)},
        "block_topk": {"ms": round(g["ms_topk"], 4),
                       "gbs": round(topk_bytes / (g["ms_topk"] * 1e-3) / 1e9, 1),
                       "frac_hbm": round(topk_bytes / (g["ms_topk"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
        "sparse_attn": {"ms": round(g["ms_attn"], 4),
                        "tflops": round(f_attn / (g["ms_attn"] * 1e-3) / 1e12, 1),
                        "frac_mfma": round(f_attn / (g["ms_attn"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)},
    }
    if w.name == "prefill_128k":  # HBM rate of the attention stage from the recorded counter bytes
        stages["sparse_attn"]["hbm_bytes"] = ATTN_TRAFFIC_BYTES
        stages["sparse_attn"]["hbm_gbs"] = round(ATTN_TRAFFIC_BYTES / (g["ms_attn"] * 1e-3) / 1e9, 1)
        stages["sparse_attn"]["frac_hbm"] = round(ATTN_TRAFFIC_BYTES / (g["ms_attn"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
        stages["sparse_attn"]["frac_of_copy"] = round(ATTN_TRAFFIC_BYTES / (g["ms_attn"] * 1e-3) / 1e9 / copy_gbs, 4)
    combined = (f_idx + f_attn) / (g["ms_step"] * 1e-3) / 1e12
    line = {
        "metric": "MSA prefill tokens/s @128K; decode tokens/s @256K KV; % of roofline",
        "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(g["ms_step"], 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "n_q": w.n_q, "n_kv": w.n_kv, "h_q": w.h_q, "h_kv": w.h_kv,
                   "head_dim": w.head_dim, "index_dim": w.index_dim, "block_size": w.block_size, "topk": w.topk},
        "roofline": roofline,
        "combined_mfma_frac": round(combined / PEAK_BF16_TFLOPS, 4),
        "hbm_copy_gbs": round(copy_gbs, 1),
        "algorithmic_tflop_per_step": round((f_idx + f_attn) / 1e12, 3),
        "stages": stages,
        "wall_ms_per_step": round(g["wall_ms_step"], 4),
    }

    if not args.no_decode:
        wd = synth.WORKLOADS[args.decode_workload]
        gd = gpu_leg(wd, args.steps, args.warmup, stream, paged=not args.no_paged)
        db = decode_bytes(wd)
        line["decode"] = {
            "workload": wd.name, "tokens_per_s": round(wd.batch / (gd["ms_step"] * 1e-3), 1),
            "ms_per_step": round(gd["ms_step"], 4), "bytes_per_step": db,
            "hbm_gbs": round(db / (gd["ms_step"] * 1e-3) / 1e9, 1),
            "frac_hbm": round(db / (gd["ms_step"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "frac_of_copy": round(db / (gd["ms_step"] * 1e-3) / 1e9 / copy_gbs, 4),
            "stages_ms": {"index_scores": round(gd["ms_index"], 4), "block_topk": round(gd["ms_topk"], 4),
                          "sparse_attn": round(gd["ms_attn"], 4)},
            "graph_ms_per_step": round(gd["ms_step_graph"], 4),
            "graph_tokens_per_s": round(wd.batch / (gd["ms_step_graph"] * 1e-3), 1),
        }

    if "ms_kl" in g:
        # S = Q K^T for every head and Z = IQ IK^T for every group, over each row's tokens
        _, _, _, t_size = algorithmic_work(w)
        f_kl = 2.0 * (w.head_dim * w.h_q + w.index_dim * w.h_kv) * w.batch * float(t_size.sum())
        line["kl"] = {"ms": round(g["ms_kl"], 4), "tflops": round(f_kl / (g["ms_kl"] * 1e-3) / 1e12, 1),
                      "frac_mfma": round(f_kl / (g["ms_kl"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                      "mean_kl": round(g["kl_mean"], 5)}
        # its gradient: S for every head, then Z, d_index_k and d_index_q for every group
        f_klb = 2.0 * (w.head_dim * w.h_q + 3 * w.index_dim * w.h_kv) * w.batch * float(t_size.sum())
        line["kl_backward"] = {"ms": round(g["ms_kl_bwd"], 4),
                               "tflops": round(f_klb / (g["ms_kl_bwd"] * 1e-3) / 1e12, 1),
                               "frac_mfma": round(f_klb / (g["ms_kl_bwd"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        # dense mode: every visible token (sum over rows of p + 1)
        import numpy as np
        n_vis = float(np.sum(w.offset + np.arange(w.n_q, dtype=np.int64) + 1)) * w.batch
        f_dense = 4.0 * w.head_dim * w.h_q * n_vis
        f_dkl = 2.0 * (w.head_dim * w.h_q + w.index_dim * w.h_kv) * n_vis
        # backward: S recomputed, dP, dV, dK, dQ over each row's tokens (five products)
        f_bwd = 2.5 * f_attn
        line["backward"] = {"ms": round(g["ms_bwd"], 4), "tflops": round(f_bwd / (g["ms_bwd"] * 1e-3) / 1e12, 1),
                            "frac_mfma": round(f_bwd / (g["ms_bwd"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        line["dense"] = {
            "attn_ms": round(g["ms_dense_attn"], 3),
            "attn_tflops": round(f_dense / (g["ms_dense_attn"] * 1e-3) / 1e12, 1),
            "attn_frac_mfma": round(f_dense / (g["ms_dense_attn"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "kl_ms": round(g["ms_dense_kl"], 3),
            "kl_tflops": round(f_dkl / (g["ms_dense_kl"] * 1e-3) / 1e12, 1),
            "kl_frac_mfma": round(f_dkl / (g["ms_dense_kl"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "msa_speedup_over_dense": round(g["ms_dense_attn"] / g["ms_step"], 2)}

    if not args.no_paged:
        # the same steps with the caches in a shuffled page pool (msa_forward_v, uniform lengths)
        line["paged"] = {"prefill_ms_per_step": round(g["ms_step_paged"], 4),
                         "prefill_tokens_per_s": round(w.batch * w.n_q / (g["ms_step_paged"] * 1e-3), 1),
                         "prefill_vs_contiguous": round(g["ms_step"] / g["ms_step_paged"], 4),
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
        f8_tflops = f_idx / (gf["ms_index"] * 1e-3) / 1e12
        line["fp8_index"] = {"prefill_ms_per_step": round(gf["ms_step"], 4),
                             "prefill_tokens_per_s": round(w.batch * w.n_q / (gf["ms_step"] * 1e-3), 1),
                             "index_scores_ms": round(gf["ms_index"], 4), "index_tflops": round(f8_tflops, 1),
                             "index_frac_fp8_mfma": round(f8_tflops / PEAK_FP8_TFLOPS, 4)}
        if not args.no_decode:
            wdf = wd.replace(name=wd.name + "_fp8_index", index_dtype="fp8")
            gdf = gpu_leg(wdf, args.steps, args.warmup, stream)
            dbf = decode_bytes(wdf)
            line["fp8_index"].update({
                "decode_ms_per_step": round(gdf["ms_step"], 4),
                "decode_tokens_per_s": round(wdf.batch / (gdf["ms_step"] * 1e-3), 1),
                "decode_bytes_per_step": dbf,
                "decode_frac_hbm": round(dbf / (gdf["ms_step"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                "decode_index_ms": round(gdf["ms_index"], 4)})
        # E4M3 K/V caches (the index branch bf16), then both branches E4M3 for decode
        wk = w.replace(name=w.name + "_fp8_kv", kv_dtype="fp8")
        gk = gpu_leg(wk, args.steps, args.warmup, stream)
        line["fp8_kv"] = {"prefill_ms_per_step": round(gk["ms_step"], 4),
                          "prefill_tokens_per_s": round(w.batch * w.n_q / (gk["ms_step"] * 1e-3), 1),
                          "sparse_attn_ms": round(gk["ms_attn"], 4)}
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
                    key + "_frac_hbm": round(dbk / (gdk["ms_step"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                    key + "_attn_ms": round(gdk["ms_attn"], 4)})

    if not args.no_cpu_baseline:
        print("[bench] oracle CPU baseline", file=sys.stderr, flush=True)
        rate, spent, n_tok, threads = cpu_leg(w, args.cpu_positions)
        line["cpu_baseline"] = {"value": round(rate, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
                                "sample": f"{n_tok} query positions (stratified over the {w.n_q}-token prefill, "
                                          f"all {w.h_kv} groups / {w.h_q} heads), {spent:.1f} s of oracle time"}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
