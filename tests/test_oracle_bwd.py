"""Pins of the oracle's Main-Branch gradient (oracle_attend_bwd), CPU only.

The gradient of softmax attention over a row's token set has a closed form;
the oracle writes it out.  Pins:
  - torch autograd (fp64) through softmax attention over the same tokens, on
    random rows with several heads, blocks and a causal cut;
  - the sum rule sum_j dV_j = sum_h dO_h (each head's weights sum to one);
  - constant V (every value row equal): the output does not depend on q or k,
    so dQ = dK = 0 exactly;
  - a shift of every key by one vector leaves dQ and dV unchanged (the
    softmax is shift invariant per head and sum_j dS_j = 0);
  - linearity in dO.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth


def rand_bits(rng, shape, scale=1.0):
    return synth.f32_to_bf16((rng.standard_normal(shape) * scale).astype(np.float32))


def vals(b):
    return synth.bf16_to_f32(b).astype(np.float64)


def case(seed, n=6, G=3, d=16, n_kv=40, bk=8, k=3):
    rng = np.random.default_rng(seed)
    q, dO = rand_bits(rng, (n, G, d)), rand_bits(rng, (n, G, d))
    K, V = rand_bits(rng, (n_kv, d)), rand_bits(rng, (n_kv, d))
    pos = rng.integers(0, n_kv, size=n)
    sel = []
    for p in pos:
        loc = p // bk
        others = sorted(rng.choice(loc, size=min(k - 1, loc), replace=False).tolist()) if loc else []
        row = sorted(others + [loc])
        sel.append(row + [-1] * (k - len(row)))
    return q, dO, K, V, pos, np.array(sel, np.int32), bk, 1.0 / math.sqrt(d)


@pytest.mark.parametrize("seed", range(4))
def test_matches_torch_autograd(seed):
    q, dO, K, V, pos, sel, bk, scale = case(seed)
    dQ, dK, dV = oracle.attend_bwd(q, pos, sel, K, V, bk, scale, dO)
    Qt = torch.tensor(vals(q), requires_grad=True)
    Kt = torch.tensor(vals(K), requires_grad=True)
    Vt = torch.tensor(vals(V), requires_grad=True)
    total = 0.0
    for r, p in enumerate(pos):
        toks = [j for t in sel[r] if t >= 0 for j in range(t * bk, min((t + 1) * bk, K.shape[0])) if j <= p]
        idx = torch.tensor(toks)
        w = torch.softmax(scale * Qt[r] @ Kt[idx].T, dim=-1)
        total = total + (w @ Vt[idx] * torch.tensor(vals(dO[r]))).sum()
    total.backward()
    assert np.allclose(dQ, Qt.grad.numpy(), rtol=1e-11, atol=1e-13)
    assert np.allclose(dK, Kt.grad.numpy(), rtol=1e-11, atol=1e-13)
    assert np.allclose(dV, Vt.grad.numpy(), rtol=1e-11, atol=1e-13)


def test_value_gradient_sum_rule():
    q, dO, K, V, pos, sel, bk, scale = case(11)
    _, _, dV = oracle.attend_bwd(q, pos, sel, K, V, bk, scale, dO)
    assert np.allclose(dV.sum(axis=0), vals(dO).sum(axis=(0, 1)), rtol=1e-12, atol=1e-12)


def test_constant_values_give_zero_query_and_key_gradients():
    q, dO, K, V, pos, sel, bk, scale = case(12)
    Vc = np.tile(V[:1], (V.shape[0], 1))
    dQ, dK, _ = oracle.attend_bwd(q, pos, sel, K, Vc, bk, scale, dO)
    assert np.abs(dQ).max() < 1e-13 and np.abs(dK).max() < 1e-13


def test_key_shift_leaves_query_and_value_gradients():
    q, dO, K, V, pos, sel, bk, scale = case(13)
    shift = synth.f32_to_bf16(np.full(K.shape[1], 0.5, np.float32))
    # values on a coarse grid so that k + 0.5 stays exact in bf16
    Kc = synth.f32_to_bf16(np.round(vals(K) * 4).astype(np.float32) / 4)
    Ks = synth.f32_to_bf16((vals(Kc) + vals(shift)[None, :]).astype(np.float32))
    assert np.array_equal(vals(Ks), vals(Kc) + 0.5)
    a = oracle.attend_bwd(q, pos, sel, Kc, V, bk, scale, dO)
    b = oracle.attend_bwd(q, pos, sel, Ks, V, bk, scale, dO)
    assert np.allclose(a[0], b[0], rtol=1e-10, atol=1e-12)
    assert np.allclose(a[2], b[2], rtol=1e-10, atol=1e-12)


def test_linear_in_output_gradient():
    q, dO, K, V, pos, sel, bk, scale = case(14)
    dO2 = synth.f32_to_bf16((2 * vals(dO)).astype(np.float32))
    a = oracle.attend_bwd(q, pos, sel, K, V, bk, scale, dO)
    b = oracle.attend_bwd(q, pos, sel, K, V, bk, scale, dO2)
    for x, y in zip(a, b):
        assert np.allclose(2 * x, y, rtol=1e-12, atol=1e-14)
