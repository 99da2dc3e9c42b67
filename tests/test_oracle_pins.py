"""Pins for the fp64 oracle: checks against facts fixed by the pages and by
mathematics, not against the oracle itself.

Pages (titles as printed): "MiniMax 发布 MSA 稀疏注意力方法，开源推理内核并推出
MiniMax-M3 模型" (sections 什么是 MSA, 两个分支如何工作, 内核协同设计) and "MiniMax
lança MSA: atenção esparsa treinada em modelo de 109B parâmetros com 3 trilhões
de tokens" (section "Como funciona o MSA", item "Local Block Forçado").
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import accept

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def bf16_bits(x):
    """Exact bf16 bit patterns of values that bf16 represents exactly."""
    x = np.asarray(x, dtype=np.float32)
    b = synth.f32_to_bf16(x)
    assert np.array_equal(synth.bf16_to_f32(b), x), "value not exact in bf16"
    return b


def rand_bits(rng, shape, scale=1.0):
    return synth.f32_to_bf16((rng.standard_normal(shape) * scale).astype(np.float32))


# ---------------------------------------------------------------- hand-worked golden values
def test_golden_index_example():
    g = json.load(open(GOLDEN))["index_example"]
    ik = bf16_bits(g["ik"])
    for row in g["rows"]:
        iq = bf16_bits([row["iq"]])
        pooled = oracle.pool(iq, [row["p"]], ik, g["block_size"])
        n = len(row["pooled"])
        assert np.array_equal(pooled[0, :n], np.array(row["pooled"], float)), row["why"]
        assert np.all(np.isnan(pooled[0, n:]))
        sel = oracle.select(pooled, [row["p"]], g["block_size"], g["topk"])
        assert sel[0].tolist() == row["sel"], row["why"]


def test_golden_attend_uniform():
    g = json.load(open(GOLDEN))["attend_uniform"]
    V = bf16_bits(g["v"])
    K = bf16_bits(np.zeros_like(np.array(g["v"], float)))
    q = bf16_bits(np.ones((len(g["rows"]), 1, 2)))
    pos = [r["p"] for r in g["rows"]]
    sel = np.array([r["sel"] for r in g["rows"]], np.int32)
    out, lse = oracle.attend(q, pos, sel, K, V, g["block_size"], g["scale"])
    for i, r in enumerate(g["rows"]):
        assert np.allclose(out[i, 0], r["out"], rtol=0, atol=1e-15)
        assert abs(lse[i, 0] - math.log(r["lse_of"])) < 1e-15


def test_golden_attend_weighted():
    g = json.load(open(GOLDEN))["attend_weighted"]
    out, lse = oracle.attend(bf16_bits([[g["q"]]]), [g["p"]], np.array([g["sel"]], np.int32),
                             bf16_bits(g["k"]), bf16_bits(g["v"]), g["block_size"], math.log(3.0))
    assert np.allclose(out[0, 0], g["out"], rtol=0, atol=1e-14)
    assert abs(lse[0, 0] - math.log(g["lse_of"])) < 1e-14


# ---------------------------------------------------------------- pooling closed forms
def test_pool_one_hot_closed_form():
    """iq = e_a and ik[j] = c_j e_a give pooled[t] = max of c_j over the
    visible tokens of block t; a huge c at j = p+1 must not leak in (R2, R4)."""
    rng = np.random.default_rng(1000)
    bk, d_idx, n = 8, 16, 64
    for trial in range(20):
        a = int(rng.integers(d_idx))
        c = rng.integers(-50, 50, size=n).astype(np.float32)
        p = int(rng.integers(0, n - 1))
        c[p + 1] = 1000.0
        ik = np.zeros((n, d_idx), np.float32)
        ik[:, a] = c
        iq = np.zeros((1, d_idx), np.float32)
        iq[0, a] = 1.0
        pooled = oracle.pool(bf16_bits(iq), [p], bf16_bits(ik), bk)
        local = p // bk
        for t in range(local + 1):
            expect = c[t * bk:min((t + 1) * bk, p + 1)].max()
            assert pooled[0, t] == expect
        assert np.all(np.isnan(pooled[0, local + 1:]))


def test_pool_orthogonal_groups():
    """Keys built from two orthogonal directions: a query along direction 0
    sees only the first component (pins the contraction index)."""
    bk, n = 4, 16
    ik = np.zeros((n, 8), np.float32)
    ik[:, 0] = np.arange(n)            # grows with j
    ik[:, 1] = -np.arange(n) * 3       # falls with j
    for p in [3, 7, 15]:
        pooled0 = oracle.pool(bf16_bits([[1, 0, 0, 0, 0, 0, 0, 0]]), [p], bf16_bits(ik), bk)[0]
        pooled1 = oracle.pool(bf16_bits([[0, 1, 0, 0, 0, 0, 0, 0]]), [p], bf16_bits(ik), bk)[0]
        for t in range(p // bk + 1):
            last = min((t + 1) * bk, p + 1) - 1
            assert pooled0[t] == last
            assert pooled1[t] == -3 * t * bk


# ---------------------------------------------------------------- P1 brute force
def brute_force_select(scores, local, k):
    """Enumerate every (k-1)-subset of the non-local candidates; keep the ones
    where each member beats each non-member in (score desc, index asc)."""
    cands = list(range(local))
    winners = []
    for sub in itertools.combinations(cands, k - 1):
        s = set(sub)
        ok = all((scores[a], -a) > (scores[c], -c) for a in s for c in cands if c not in s)
        if ok:
            winners.append(sorted(s) + [local])
    return winners


@pytest.mark.parametrize("seed", range(1000, 1040))
def test_select_brute_force(seed):
    rng = np.random.default_rng(seed)
    k = int(rng.integers(2, 7))
    local = int(rng.integers(k, 13))
    bk = int(rng.choice([1, 2, 4, 8]))
    p = local * bk + int(rng.integers(0, bk))
    ties = seed % 2 == 0
    scores = (rng.integers(-3, 4, size=local + 1).astype(float) if ties else rng.standard_normal(local + 1))
    pooled = np.full((1, local + 1), np.nan)
    pooled[0, :] = scores
    sel = oracle.select(pooled, [p], bk, k)[0].tolist()
    winners = brute_force_select(scores, local, k)
    assert len(winners) == 1
    assert sel == winners[0]
    if not ties:
        best = max(itertools.combinations(range(local), k - 1), key=lambda s: sum(scores[a] for a in s))
        assert sorted(best) + [local] == sel


def test_select_few_blocks_pads():
    """At most k visible blocks: all are kept, the rest of the row is -1 (R6)."""
    for local in range(0, 5):
        pooled = np.zeros((1, 8))
        sel = oracle.select(pooled, [local * 4 + 1], 4, 5)[0]
        assert sel.tolist() == list(range(local + 1)) + [-1] * (5 - local - 1)


# ---------------------------------------------------------------- P2 exp-free invariance
@pytest.mark.parametrize("seed", range(1100, 1110))
def test_select_exp_free_invariance(seed):
    """Top-k on softmax(P) equals top-k on raw P (softmax keeps the order)."""
    rng = np.random.default_rng(seed)
    n = 300
    local = np.arange(n) // 2 + 20
    pooled = rng.uniform(-20, 20, size=(n, local.max() + 1))
    soft = np.full_like(pooled, np.nan)
    for r in range(n):
        x = pooled[r, :local[r] + 1]
        e = np.exp(x - x.max())
        soft[r, :local[r] + 1] = e / e.sum()
    pos = local * 8 + 3
    assert np.array_equal(oracle.select(pooled, pos, 8, 16), oracle.select(soft, pos, 8, 16))


# ---------------------------------------------------------------- P3 forced local
def test_forced_local_adversarial():
    """Local block's index keys set to -10x the others' magnitude: its pooled
    score is the row minimum, yet it is selected as the last valid entry."""
    rng = np.random.default_rng(1200)
    bk, d_idx, n = 16, 32, 512
    ik = rng.standard_normal((n, d_idx)).astype(np.float32)
    iq = np.abs(rng.standard_normal((1, d_idx))).astype(np.float32)
    ik = np.abs(ik)
    for p in range(bk * 8, n, 37):
        local = p // bk
        ik2 = ik.copy()
        ik2[local * bk:(local + 1) * bk] *= -10
        pooled = oracle.pool(synth.f32_to_bf16(iq), [p], synth.f32_to_bf16(ik2), bk)
        assert pooled[0, local] == np.nanmin(pooled[0, :local + 1])
        sel = oracle.select(pooled, [p], bk, 6)[0]
        assert accept.structure_ok(sel, local, 6)
        assert sel[-1] == local


# ---------------------------------------------------------------- P4 dense equivalence
def _sdpa_ref(q_rows, pos, K, V, scale):
    """Causal GQA attention via torch's scaled_dot_product_attention (fp64 CPU)."""
    qf = torch.from_numpy(synth.bf16_to_f32(q_rows).astype(np.float64))     # [n, G, d]
    kf = torch.from_numpy(synth.bf16_to_f32(K).astype(np.float64))          # [n_kv, d]
    vf = torch.from_numpy(synth.bf16_to_f32(V).astype(np.float64))
    n, G, d = qf.shape
    mask = torch.from_numpy(np.arange(K.shape[0])[None, :] <= np.asarray(pos)[:, None])  # [n, n_kv]
    out = torch.nn.functional.scaled_dot_product_attention(
        qf.permute(1, 0, 2)[None], kf[None, None].expand(1, G, -1, -1), vf[None, None].expand(1, G, -1, -1),
        attn_mask=mask[None, None].expand(1, G, -1, -1), scale=scale)
    return out[0].permute(1, 0, 2).numpy()


def test_dense_gqa_matches_torch_sdpa():
    rng = np.random.default_rng(1300)
    n_kv, d, G = 200, 32, 3
    K, V = rand_bits(rng, (n_kv, d)), rand_bits(rng, (n_kv, d))
    pos = np.array([0, 1, 5, 63, 64, 127, 150, 199])
    q = rand_bits(rng, (len(pos), G, d))
    out, lse = oracle.dense_gqa(q, pos, K, V, 0.17)
    ref = _sdpa_ref(q, pos, K, V, 0.17)
    assert np.max(np.abs(out - ref)) < 1e-12
    # lse closed form for the first row: a single token
    qk = synth.bf16_to_f32(q[0, :, :]).astype(np.float64) @ synth.bf16_to_f32(K[0]).astype(np.float64)
    assert np.allclose(lse[0], 0.17 * qk, atol=1e-13)


@pytest.mark.parametrize("bk,k,n_kv", [(8, 4, 32), (16, 8, 100), (4, 16, 64), (32, 2, 64)])
def test_sparse_equals_dense_when_budget_covers_all(bk, k, n_kv):
    """k*Bk >= n_kv: every visible block is selected and the sparse result is
    dense causal GQA (to 1e-12)."""
    assert k * bk >= n_kv
    rng = np.random.default_rng(1400 + bk)
    G, d, d_idx = 4, 32, 16
    K, V = rand_bits(rng, (n_kv, d)), rand_bits(rng, (n_kv, d))
    ik = rand_bits(rng, (n_kv, d_idx))
    pos = np.arange(n_kv)
    iq = rand_bits(rng, (n_kv, d_idx))
    q = rand_bits(rng, (n_kv, G, d))
    pooled = oracle.pool(iq, pos, ik, bk)
    sel = oracle.select(pooled, pos, bk, k)
    for r in range(n_kv):
        assert sel[r][sel[r] >= 0].tolist() == list(range(pos[r] // bk + 1))
    out, lse = oracle.attend(q, pos, sel, K, V, bk, 0.2)
    dout, dlse = oracle.dense_gqa(q, pos, K, V, 0.2)
    assert np.max(np.abs(out - dout)) <= 1e-12
    assert np.max(np.abs(lse - dlse)) <= 1e-12


# ---------------------------------------------------------------- P5 k = 1
def test_k1_is_attention_within_own_block():
    rng = np.random.default_rng(1500)
    bk, n_kv, G, d, d_idx = 16, 96, 2, 32, 8
    K, V = rand_bits(rng, (n_kv, d)), rand_bits(rng, (n_kv, d))
    pos = np.arange(n_kv)
    pooled = oracle.pool(rand_bits(rng, (n_kv, d_idx)), pos, rand_bits(rng, (n_kv, d_idx)), bk)
    sel = oracle.select(pooled, pos, bk, 1)
    assert np.array_equal(sel[:, 0], pos // bk)
    q = rand_bits(rng, (n_kv, G, d))
    out, _ = oracle.attend(q, pos, sel, K, V, bk, 0.3)
    for r in range(n_kv):
        j0 = (pos[r] // bk) * bk
        ref = _sdpa_ref(q[r:r + 1], [pos[r] - j0], K[j0:pos[r] + 1], V[j0:pos[r] + 1], 0.3)
        assert np.max(np.abs(out[r] - ref[0])) < 1e-12


# ---------------------------------------------------------------- P6 p = 0
def test_first_position_returns_v0():
    rng = np.random.default_rng(1600)
    K, V = rand_bits(rng, (64, 32)), rand_bits(rng, (64, 32))
    q = rand_bits(rng, (1, 3, 32))
    out, lse = oracle.attend(q, [0], np.array([[0, -1, -1]], np.int32), K, V, 16, 0.5)
    v0 = synth.bf16_to_f32(V[0]).astype(np.float64)
    assert np.array_equal(out[0], np.broadcast_to(v0, (3, 32)))
    qk = synth.bf16_to_f32(q[0]).astype(np.float64) @ synth.bf16_to_f32(K[0]).astype(np.float64)
    assert np.allclose(lse[0], 0.5 * qk, rtol=0, atol=1e-14)


# ---------------------------------------------------------------- P7 merge invariance
@pytest.mark.parametrize("seed", range(1700, 1705))
def test_merge_of_partitions_equals_whole(seed):
    """Attention over T equals the LSE merge of attention over the parts of
    any partition of T into block subsets (the two-stage forward)."""
    rng = np.random.default_rng(seed)
    bk, n_kv, G, d, k = 16, 320, 4, 32, 8
    K, V = rand_bits(rng, (n_kv, d)), rand_bits(rng, (n_kv, d))
    p = int(rng.integers(bk * k, n_kv))
    local = p // bk
    blocks = sorted(rng.choice(local, size=k - 1, replace=False).tolist()) + [local]
    q = rand_bits(rng, (1, G, d))
    whole, wlse = oracle.attend(q, [p], np.array([blocks], np.int32), K, V, bk, 0.1)
    nparts = int(rng.integers(2, k + 1))
    label = rng.integers(0, nparts, size=k)
    label[:nparts] = np.arange(nparts)
    o_parts, l_parts = [], []
    for s in range(nparts):
        part = [b for b, l in zip(blocks, label) if l == s]
        sel = np.array([part + [-1] * (k - len(part))], np.int32)
        o, l = oracle.attend(q, [p], sel, K, V, bk, 0.1)
        o_parts.append(o[0])
        l_parts.append(l[0])
    o_parts = np.stack(o_parts, axis=1)   # [G, P, d]
    l_parts = np.stack(l_parts, axis=1)   # [G, P]
    mo, ml = oracle.merge(o_parts, l_parts)
    assert np.max(np.abs(mo - whole[0])) <= 1e-13
    assert np.max(np.abs(ml - wlse[0])) <= 1e-13


def test_merge_ignores_empty_parts():
    o = np.random.default_rng(1).standard_normal((2, 3, 4))
    l = np.array([[0.5, -np.inf, 1.0], [-np.inf, 2.0, -np.inf]])
    mo, ml = oracle.merge(o, l)
    w = np.exp(np.array([0.5, 1.0]) - np.log(np.exp(0.5) + np.exp(1.0)))
    assert np.allclose(mo[0], w[0] * o[0, 0] + w[1] * o[0, 2], atol=1e-15)
    assert np.allclose(mo[1], o[1, 1], atol=1e-15) and abs(ml[1] - 2.0) < 1e-15


# ---------------------------------------------------------------- P8 decode == prefill row
def test_decode_equals_last_prefill_row():
    w = synth.Workload("tiny", 1, 512, 512, 8, 2, head_dim=32, index_dim=16, block_size=16, topk=4, seed=1800)
    wd = w.replace(n_q=1)     # bottom-right aligned: p = n_kv - 1
    for g in range(2):
        full = oracle.forward_rows(w, 0, g, [511])
        # the decode workload's query row 0 is a different generator row; give it the same inputs
        x = oracle.inputs_for_rows(w, 0, g, [511])
        assert wd.offset + 0 == x["pos"][0]
        pooled = oracle.pool(x["iq"], [wd.offset], x["ik"], wd.block_size)
        sel = oracle.select(pooled, [wd.offset], wd.block_size, wd.topk)
        assert np.array_equal(sel, full["sel"])


def test_chunked_rows_equal_full_prefill_rows():
    """A chunk of queries at an offset computes the matching rows of the full prefill."""
    rng = np.random.default_rng(1810)
    bk, n_kv, d_idx = 8, 256, 16
    ik = rand_bits(rng, (n_kv, d_idx))
    iq = rand_bits(rng, (n_kv, d_idx))
    pos = np.arange(n_kv)
    full = oracle.select(oracle.pool(iq, pos, ik, bk), pos, bk, 5)
    chunk = oracle.select(oracle.pool(iq[200:], pos[200:], ik, bk), pos[200:], bk, 5)
    assert np.array_equal(full[200:], chunk)


# ---------------------------------------------------------------- P9 scale & permutation
def test_index_scale_and_permutation_invariance():
    rng = np.random.default_rng(1900)
    bk, n_kv, d_idx, k = 8, 200, 16, 6
    ik = rand_bits(rng, (n_kv, d_idx))
    iq = rand_bits(rng, (n_kv, d_idx))
    pos = np.arange(n_kv)
    p1 = oracle.pool(iq, pos, ik, bk)
    iq2 = synth.f32_to_bf16(synth.bf16_to_f32(iq) * 2)        # exact in bf16
    p2 = oracle.pool(iq2, pos, ik, bk)
    assert np.array_equal(np.nan_to_num(p2), np.nan_to_num(2 * p1))
    assert np.array_equal(oracle.select(p1, pos, bk, k), oracle.select(p2, pos, bk, k))
    perm = rng.permutation(d_idx)                              # permuting the index dim
    p3 = oracle.pool(iq[:, perm], pos, ik[:, perm], bk)
    assert np.allclose(np.nan_to_num(p3), np.nan_to_num(p1), rtol=1e-14, atol=1e-12)


def test_head_permutation_within_group():
    rng = np.random.default_rng(1910)
    bk, n_kv, G, d = 8, 128, 5, 32
    K, V = rand_bits(rng, (n_kv, d)), rand_bits(rng, (n_kv, d))
    pos = np.arange(40, 128, 7)
    sel = np.array([[0, 2, p // bk, -1] for p in pos], np.int32)
    q = rand_bits(rng, (len(pos), G, d))
    perm = rng.permutation(G)
    o1, l1 = oracle.attend(q, pos, sel, K, V, bk, 0.2)
    o2, l2 = oracle.attend(q[:, perm], pos, sel, K, V, bk, 0.2)
    assert np.array_equal(o2, o1[:, perm]) and np.array_equal(l2, l1[:, perm])


# ---------------------------------------------------------------- P10 all-equal scores
def test_all_equal_scores_pick_lowest_blocks():
    bk, n_kv, d_idx, k = 8, 256, 16, 5
    ik = bf16_bits(np.ones((n_kv, d_idx)))
    pos = np.arange(0, n_kv, 3)
    iq = bf16_bits(np.full((len(pos), d_idx), 0.5))
    sel = oracle.select(oracle.pool(iq, pos, ik, bk), pos, bk, k)
    for r, p in enumerate(pos):
        local = p // bk
        exp = list(range(local + 1)) + [-1] * (k - local - 1) if local + 1 <= k else list(range(k - 1)) + [local]
        assert sel[r].tolist() == exp


def test_signed_zero_ties():
    """-0.0 and +0.0 are equal scores: the lower block index wins (R7)."""
    pooled = np.array([[-0.0, 0.0, -1.0, 0.0, -0.0, 5.0]])
    sel = oracle.select(pooled, [5 * 4], 4, 3)[0].tolist()
    assert sel == [0, 1, 5]
    pooled = np.array([[0.0, -0.0, -1.0, 5.0]])
    assert oracle.select(pooled, [3 * 4], 4, 2)[0].tolist() == [0, 3]


# ---------------------------------------------------------------- acceptance rules
def test_acceptance_rules():
    P = np.array([5.0, 4.0, 3.0, 2.9999, 1.0, 0.0])   # local = 5
    assert accept.gap_rel(P, 5, 4) == pytest.approx((3.0 - 2.9999) / 3.0)
    assert accept.eps_valid([0, 1, 3, 5], P, 5, 4)     # swap inside the gap is fine
    assert not accept.eps_valid([0, 1, 4, 5], P, 5, 4)
    assert not accept.structure_ok([0, 1, 5, 3], 5, 4)
    assert not accept.structure_ok([0, 1, 2, -1], 5, 4)
    assert accept.structure_ok([0, 1, -1, -1], 1, 4)
    assert accept.gap_rel(P, 2, 4) == float("inf")


# ---------------------------------------------------------------- argument errors
def test_oracle_rejects_bad_arguments():
    with pytest.raises(ValueError):
        oracle.pool(np.zeros((1, 4), np.uint16), [10], np.zeros((8, 4), np.uint16), 4)   # p >= n_kv
    with pytest.raises(ValueError):
        oracle.select(np.zeros((1, 4)), [3], 1, 0)                                      # k < 1


# ---------------------------------------------------------------- the matrix-product form of the pool
def test_pool_mm_golden_and_closed_forms():
    """pool_mm (fp64 library product + block max) reproduces the hand-worked
    pooled values and the one-hot closed form exactly (small integers: every
    summation order is exact)."""
    g = json.load(open(GOLDEN))["index_example"]
    ik = bf16_bits(g["ik"])
    for row in g["rows"]:
        pooled = oracle.pool_mm(bf16_bits([row["iq"]]), [row["p"]], ik, g["block_size"])
        n = len(row["pooled"])
        assert np.array_equal(pooled[0, :n], np.array(row["pooled"], float)), row["why"]
        assert np.all(np.isnan(pooled[0, n:]))
    rng = np.random.default_rng(1900)
    bk, d_idx, n = 8, 16, 200
    for trial in range(10):
        a = int(rng.integers(d_idx))
        c = rng.integers(-50, 50, size=n).astype(np.float32)
        p = int(rng.integers(0, n - 1))
        c[p + 1] = 1000.0   # the first invisible key must not leak into the local block
        ik1 = np.zeros((n, d_idx), np.float32)
        ik1[:, a] = c
        iq = np.zeros((1, d_idx), np.float32)
        iq[0, a] = 1.0
        pooled = oracle.pool_mm(bf16_bits(iq), [p], bf16_bits(ik1), bk, keys_per_step=24)   # several key steps
        for t in range(p // bk + 1):
            assert pooled[0, t] == c[t * bk:min((t + 1) * bk, p + 1)].max()
        assert np.all(np.isnan(pooled[0, p // bk + 1:]))


@pytest.mark.parametrize("n_kv,bk,step", [(1000, 128, 256), (4096, 128, 16384), (333, 16, 48)])
def test_pool_mm_equals_plain_loops(n_kv, bk, step):
    """On random bf16 rows (ragged tail, every position class) the product
    form equals the plain loops of oracle_pool to fp64 rounding."""
    rng = np.random.default_rng(1901 + n_kv)
    d_idx = 64
    ik = rand_bits(rng, (n_kv, d_idx))
    pos = np.unique(np.concatenate([[0, bk - 1, bk, n_kv - 1], rng.integers(0, n_kv, 60)]))
    iq = rand_bits(rng, (len(pos), d_idx))
    a = oracle.pool(iq, pos, ik, bk)
    b = oracle.pool_mm(iq, pos, ik, bk, keys_per_step=step)
    assert np.array_equal(np.isnan(a), np.isnan(b))
    fin = ~np.isnan(a)
    assert np.max(np.abs(a[fin] - b[fin]) / np.maximum(np.abs(a[fin]), 1.0)) < 1e-13


def test_pool_mm_fp8_equals_plain_loops():
    rng = np.random.default_rng(1902)
    n_kv, bk, d_idx = 700, 128, 128
    ik = synth.to_e4m3(rand_bits(rng, (n_kv, d_idx)))
    pos = np.array([0, 127, 128, 300, 699])
    iq = synth.to_e4m3(rand_bits(rng, (len(pos), d_idx)))
    a = oracle.pool_f8(iq, pos, ik, bk)
    b = oracle.pool_mm(iq, pos, ik, bk, keys_per_step=256)
    fin = ~np.isnan(a)
    assert np.array_equal(fin, ~np.isnan(b))
    assert np.max(np.abs(a[fin] - b[fin]) / np.maximum(np.abs(a[fin]), 1.0)) < 1e-13
