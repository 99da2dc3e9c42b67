"""Pins of the oracle's KL alignment term (oracle_kl), CPU only.

Page "MiniMax 发布 MSA 稀疏注意力方法，开源推理内核并推出 MiniMax-M3 模型", section
MSA 如何训练: the loss matches the Index Branch's distribution to the Main
Branch's attention, the teacher being the Main Branch's group-averaged
distribution over the selected tokens.  Reading R14: the student is the
softmax of the raw index scores over the same tokens.  Pins:
  - a two-token row worked out by hand;
  - KL = 0 when the student reproduces the teacher (G = 1, iq = scale * q,
    ik = k), and > 0 otherwise (Gibbs' inequality);
  - a group of identical heads equals one head;
  - invariance to the order of the group's heads and to a shift of every
    student logit;
  - torch's softmax and kl_div on the same tokens (a library computation).
The teacher on its own (oracle_kl_teacher, which the stored-teacher backward
is checked against): a hand-worked row, the weights of a row summing to 1 over
T and 0 elsewhere, torch's head-averaged softmax, and the KL rebuilt from it
and the student equal to oracle_kl.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth


def bf16_bits(x):
    x = np.asarray(x, dtype=np.float32)
    b = synth.f32_to_bf16(x)
    assert np.array_equal(synth.bf16_to_f32(b), x), "value not exact in bf16"
    return b


def rand_bits(rng, shape, scale=1.0):
    return synth.f32_to_bf16((rng.standard_normal(shape) * scale).astype(np.float32))


def test_two_tokens_by_hand():
    # keys 0, 1 visible to the query at p = 1 (Bk = 2, one block).  Teacher (G = 1,
    # scale ln 3): scores 0 and ln 3 -> p = (1/4, 3/4).  Student: index scores 0 and 0
    # -> s = (1/2, 1/2).  KL = 1/4 ln(1/2) + 3/4 ln(3/2).
    q = bf16_bits([[[1.0, 0.0]]])
    K = bf16_bits([[0.0, 1.0], [1.0, 0.0]])
    iq = bf16_bits([[1.0, 1.0]])
    ik = bf16_bits([[1.0, -1.0], [-1.0, 1.0]])
    got = oracle.kl(q, [1], np.array([[0]], np.int32), K, iq, ik, 2, math.log(3.0))[0]
    want = 0.25 * math.log(0.5) + 0.75 * math.log(1.5)
    assert abs(got - want) < 1e-15


def test_student_equal_to_teacher_gives_zero():
    rng = np.random.default_rng(5)
    n_kv, d, bk = 40, 8, 4
    q = rand_bits(rng, (6, 1, d))
    K = rand_bits(rng, (n_kv, d))
    pos = rng.integers(0, n_kv, size=6)
    sel = np.array([[t for t in range(p // bk + 1)][-3:] + [-1] * (3 - len([t for t in range(p // bk + 1)][-3:]))
                    for p in pos], np.int32)
    # softmax scale 1: the student's logits iq . ik equal the teacher's scale * q . k
    got = oracle.kl(q, pos, sel, K, q[:, 0, :], K, bk, 1.0)
    assert np.all(np.abs(got) < 1e-12)


@pytest.mark.parametrize("seed", range(4))
def test_kl_is_positive_otherwise(seed):
    rng = np.random.default_rng(100 + seed)
    n_kv, d, di, bk, G = 64, 16, 8, 8, 4
    q = rand_bits(rng, (10, G, d))
    K = rand_bits(rng, (n_kv, d))
    iq = rand_bits(rng, (10, di))
    ik = rand_bits(rng, (n_kv, di))
    pos = rng.integers(1, n_kv, size=10)
    sel = np.array([sorted(set([p // bk, 0]))[:2] + [-1] * (2 - len(set([p // bk, 0]))) for p in pos], np.int32)
    got = oracle.kl(q, pos, sel, K, iq, ik, bk, 1.0 / math.sqrt(d))
    assert np.all(got > 0)


def test_identical_heads_equal_one_head_and_head_order_is_irrelevant():
    rng = np.random.default_rng(7)
    n_kv, d, di, bk = 50, 8, 8, 5
    q1 = rand_bits(rng, (5, 1, d))
    K, iq, ik = rand_bits(rng, (n_kv, d)), rand_bits(rng, (5, di)), rand_bits(rng, (n_kv, di))
    pos = np.array([4, 17, 30, 41, 49])
    sel = np.array([[0, p // bk, -1] if p // bk > 0 else [0, -1, -1] for p in pos], np.int32)
    one = oracle.kl(q1, pos, sel, K, iq, ik, bk, 0.5)
    four = oracle.kl(np.repeat(q1, 4, axis=1), pos, sel, K, iq, ik, bk, 0.5)
    assert np.allclose(one, four, rtol=1e-13, atol=1e-15)
    qg = rand_bits(rng, (5, 3, d))
    a = oracle.kl(qg, pos, sel, K, iq, ik, bk, 0.5)
    b = oracle.kl(qg[:, [2, 0, 1], :], pos, sel, K, iq, ik, bk, 0.5)
    assert np.allclose(a, b, rtol=1e-13, atol=1e-15)


def test_student_shift_invariance():
    # an extra index dim with iq = 1 and the same key value for every token adds a
    # constant to every student logit: the softmax, and the KL, do not change
    rng = np.random.default_rng(9)
    n_kv, d, di, bk = 32, 8, 7, 4
    q, K = rand_bits(rng, (4, 2, d)), rand_bits(rng, (n_kv, d))
    iq, ik = rand_bits(rng, (4, di)), rand_bits(rng, (n_kv, di))
    pos = np.array([3, 12, 20, 31])
    sel = np.array([[0, 1, p // bk] if p // bk > 1 else [0, 1, -1] for p in pos], np.int32)
    sel = np.where(sel > pos[:, None] // bk, -1, sel).astype(np.int32)
    base = oracle.kl(q, pos, sel, K, iq, ik, bk, 0.3)
    iq2 = np.concatenate([iq, bf16_bits(np.ones((4, 1)))], axis=1)
    ik2 = np.concatenate([ik, bf16_bits(np.full((n_kv, 1), 2.5))], axis=1)
    shifted = oracle.kl(q, pos, sel, K, iq2, ik2, bk, 0.3)
    assert np.allclose(base, shifted, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("seed", range(3))
def test_matches_torch_softmax_and_kl_div(seed):
    rng = np.random.default_rng(200 + seed)
    n_kv, d, di, bk, G, k = 96, 16, 16, 8, 4, 3
    n = 12
    q, K = rand_bits(rng, (n, G, d)), rand_bits(rng, (n_kv, d))
    iq, ik = rand_bits(rng, (n, di)), rand_bits(rng, (n_kv, di))
    pos = rng.integers(0, n_kv, size=n)
    sel = []
    for p in pos:
        loc = p // bk
        others = sorted(rng.choice(loc, size=min(k - 1, loc), replace=False).tolist()) if loc else []
        row = sorted(others + [loc])
        sel.append(row + [-1] * (k - len(row)))
    sel = np.array(sel, np.int32)
    scale = 1.0 / math.sqrt(d)
    got = oracle.kl(q, pos, sel, K, iq, ik, bk, scale)
    f = lambda b: torch.from_numpy(synth.bf16_to_f32(b).astype(np.float64))
    Qt, Kt, IQ, IK = f(q), f(K), f(iq), f(ik)
    for r in range(n):
        toks = [j for t in sel[r] if t >= 0 for j in range(t * bk, min((t + 1) * bk, n_kv)) if j <= pos[r]]
        idx = torch.tensor(toks)
        teacher = torch.softmax(scale * Qt[r] @ Kt[idx].T, dim=-1).mean(dim=0)
        log_student = torch.log_softmax(IQ[r] @ IK[idx].T, dim=-1)
        want = torch.nn.functional.kl_div(log_student, teacher, reduction="sum").item()
        assert abs(got[r] - want) < 1e-12 * max(1.0, abs(want))


def test_teacher_by_hand():
    # the two-token row of test_two_tokens_by_hand: weights (1/4, 3/4); a third key
    # past the position gets 0
    q = bf16_bits([[[1.0, 0.0]]])
    K = bf16_bits([[0.0, 1.0], [1.0, 0.0], [1.0, 1.0]])
    t = oracle.kl_teacher(q, [1], np.array([[0, 1]], np.int32), K, 2, math.log(3.0))
    assert np.allclose(t[0], [0.25, 0.75, 0.0], rtol=0, atol=1e-15)


@pytest.mark.parametrize("seed", range(3))
def test_teacher_sums_to_one_and_matches_torch(seed):
    rng = np.random.default_rng(400 + seed)
    n_kv, d, di, bk, G, k, n = 96, 16, 16, 8, 4, 3, 12
    q, K = rand_bits(rng, (n, G, d)), rand_bits(rng, (n_kv, d))
    iq, ik = rand_bits(rng, (n, di)), rand_bits(rng, (n_kv, di))
    pos = rng.integers(0, n_kv, size=n)
    sel = []
    for p in pos:
        loc = p // bk
        others = sorted(rng.choice(loc, size=min(k - 1, loc), replace=False).tolist()) if loc else []
        row = sorted(others + [loc])
        sel.append(row + [-1] * (k - len(row)))
    sel = np.array(sel, np.int32)
    scale = 1.0 / math.sqrt(d)
    t = oracle.kl_teacher(q, pos, sel, K, bk, scale)
    kl = oracle.kl(q, pos, sel, K, iq, ik, bk, scale)
    f = lambda b: torch.from_numpy(synth.bf16_to_f32(b).astype(np.float64))
    Qt, Kt, IQ, IK = f(q), f(K), f(iq), f(ik)
    for r in range(n):
        toks = [j for tb in sel[r] if tb >= 0 for j in range(tb * bk, min((tb + 1) * bk, n_kv)) if j <= pos[r]]
        outside = np.ones(n_kv, bool)
        outside[toks] = False
        assert np.all(t[r][outside] == 0.0)
        assert abs(t[r].sum() - 1.0) < 1e-13
        idx = torch.tensor(toks)
        want = torch.softmax(scale * Qt[r] @ Kt[idx].T, dim=-1).mean(dim=0).numpy()
        assert np.allclose(t[r][toks], want, rtol=1e-13, atol=1e-16)
        # kl = sum t ln t - sum t z + ln sum exp z over T, with the teacher above
        z = (IQ[r] @ IK[idx].T).numpy()
        tt = t[r][toks]
        nz = tt > 0
        rebuilt = np.sum(tt[nz] * np.log(tt[nz])) - np.sum(tt * z) + (z.max() + np.log(np.exp(z - z.max()).sum()))
        assert abs(rebuilt - kl[r]) < 1e-12 * max(1.0, abs(kl[r]))


# ---------------------------------------------------------------- gradient (teacher detached)
def _kl_case(seed):
    rng = np.random.default_rng(seed)
    n_kv, d, di, bk, G, k, n = 64, 16, 8, 8, 4, 3, 9
    q, K = rand_bits(rng, (n, G, d)), rand_bits(rng, (n_kv, d))
    iq, ik = rand_bits(rng, (n, di)), rand_bits(rng, (n_kv, di))
    pos = rng.integers(0, n_kv, size=n)
    sel = []
    for p in pos:
        loc = p // bk
        others = sorted(rng.choice(loc, size=min(k - 1, loc), replace=False).tolist()) if loc else []
        row = sorted(others + [loc])
        sel.append(row + [-1] * (k - len(row)))
    return q, K, iq, ik, pos, np.array(sel, np.int32), bk, 1.0 / math.sqrt(d), rng.standard_normal(n)


@pytest.mark.parametrize("seed", range(3))
def test_kl_gradient_matches_torch_autograd_with_detached_teacher(seed):
    q, K, iq, ik, pos, sel, bk, scale, w = _kl_case(300 + seed)
    d_iq, d_ik = oracle.kl_bwd(q, pos, sel, K, iq, ik, bk, scale, w)
    f = lambda b: torch.from_numpy(synth.bf16_to_f32(b).astype(np.float64))
    Qt, Kt = f(q), f(K)
    IQ = f(iq).requires_grad_(True)
    IK = f(ik).requires_grad_(True)
    loss = 0.0
    for r in range(len(pos)):
        toks = [j for t in sel[r] if t >= 0 for j in range(t * bk, min((t + 1) * bk, K.shape[0])) if j <= pos[r]]
        idx = torch.tensor(toks)
        teacher = torch.softmax(scale * Qt[r] @ Kt[idx].T, dim=-1).mean(dim=0).detach()
        log_student = torch.log_softmax(IQ[r] @ IK[idx].T, dim=-1)
        loss = loss + w[r] * torch.nn.functional.kl_div(log_student, teacher, reduction="sum")
    loss.backward()
    assert np.allclose(d_iq, IQ.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert np.allclose(d_ik, IK.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_kl_gradient_ignores_a_common_shift_of_the_index_keys():
    # sum_j (s_j - t_j) = 0: shifting every index key by one vector leaves d_iq unchanged
    q, K, iq, ik, pos, sel, bk, scale, w = _kl_case(310)
    ikc = synth.f32_to_bf16(np.round(synth.bf16_to_f32(ik) * 4).astype(np.float32) / 4)
    iks = synth.f32_to_bf16((synth.bf16_to_f32(ikc) + 0.25).astype(np.float32))
    a, _ = oracle.kl_bwd(q, pos, sel, K, iq, ikc, bk, scale, w)
    # the shift changes every logit of a row by the same amount (0.25 * sum(iq)), so s and t are unchanged
    b, _ = oracle.kl_bwd(q, pos, sel, K, iq, iks, bk, scale, w)
    assert np.allclose(a, b, rtol=1e-10, atol=1e-12)


def test_kl_gradient_vanishes_when_student_equals_teacher():
    rng = np.random.default_rng(320)
    n_kv, d, bk = 40, 8, 4
    q = rand_bits(rng, (6, 1, d))
    K = rand_bits(rng, (n_kv, d))
    pos = rng.integers(0, n_kv, size=6)
    sel = np.array([[t for t in range(p // bk + 1)][-3:] + [-1] * (3 - len([t for t in range(p // bk + 1)][-3:]))
                    for p in pos], np.int32)
    d_iq, d_ik = oracle.kl_bwd(q, pos, sel, K, q[:, 0, :], K, bk, 1.0)
    assert np.abs(d_iq).max() < 1e-12 and np.abs(d_ik).max() < 1e-12
