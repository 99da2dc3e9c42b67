"""Pins of the oracle's FP8 (OCP E4M3) index-branch functions, CPU only.

The pages say the released kernels take FP8 index inputs without naming the
format; the oracle reads it as OCP E4M3 (1 sign, 4 exponent bits with bias 7,
3 mantissa bits, no infinities, NaN = all ones).  Pins:
  - the decoder against torch's float8_e4m3fn on all 256 codes (an
    independent implementation) and against values worked out by hand from
    the format's definition;
  - pool_f8 against the already pinned bf16 pool: every E4M3 value is exactly
    a bf16 value, so the two must agree bit for bit on the same numbers;
  - a hand-worked pooled example with a subnormal, the largest finite value
    and a causal cut.
"""
import numpy as np
import pytest

import oracle
import synth


def test_e4m3_decoder_matches_torch_on_every_code():
    torch = pytest.importorskip("torch")
    c = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_decode(c)
    ref = torch.from_numpy(c.copy()).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6), (0x30, 0.5), (0x38, 1.0),
    (0x3C, 1.5), (0x40, 2.0), (0x7E, 448.0), (0xB8, -1.0), (0xFE, -448.0), (0x80, -0.0),
])
def test_e4m3_decoder_hand_values(code, value):
    got = oracle.e4m3_decode(np.array([code], np.uint8))[0]
    assert got == value and np.signbit(got) == np.signbit(value)


@pytest.mark.parametrize("code", [0x7F, 0xFF])
def test_e4m3_nan_codes(code):
    assert np.isnan(oracle.e4m3_decode(np.array([code], np.uint8))[0])


def _bf16_bits_of(values: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of values that are exactly bf16 (checked)."""
    f = values.astype(np.float32)
    assert np.array_equal(f.astype(np.float64), values)
    bits = f.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0)
    return (bits >> 16).astype(np.uint16)


@pytest.mark.parametrize("d_idx,bk,n_kv,seed", [(64, 8, 61, 1), (128, 16, 100, 2), (16, 4, 9, 3)])
def test_pool_f8_equals_bf16_pool_on_the_same_values(d_idx, bk, n_kv, seed):
    rng = np.random.default_rng(seed)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    iq = rng.choice(finite, size=(7, d_idx)).astype(np.uint8)
    ik = rng.choice(finite, size=(n_kv, d_idx)).astype(np.uint8)
    pos = rng.integers(0, n_kv, size=7)
    a = oracle.pool_f8(iq, pos, ik, bk)
    b = oracle.pool(_bf16_bits_of(oracle.e4m3_decode(iq)), pos, _bf16_bits_of(oracle.e4m3_decode(ik)), bk)
    assert np.array_equal(np.isnan(a), np.isnan(b))
    assert np.array_equal(a[~np.isnan(a)], b[~np.isnan(b)])


def test_pool_f8_hand_worked():
    # iq = (1, -0.5); keys (2, 1), (0.5, 448), (-1, 2^-6), (4, 0); Bk = 2, query at p = 2
    iq = np.array([[0x38, 0xB0]], np.uint8)
    ik = np.array([[0x40, 0x38], [0x30, 0x7E], [0xB8, 0x08], [0x48, 0x00]], np.uint8)
    pooled = oracle.pool_f8(iq, np.array([2]), ik, 2)
    # block 0: max(2 - 0.5, 0.5 - 224) = 1.5; block 1: only key 2 is visible: -1 - 2^-7
    assert pooled[0, 0] == 1.5
    assert pooled[0, 1] == -1.0 - 2.0 ** -7


def test_kv_values_bf16_are_the_e4m3_values():
    """The oracle's view of FP8 K/V rows equals torch's own float8_e4m3fn round
    trip of the same bf16 values, and is the identity for bf16 workloads."""
    import torch
    rng = np.random.default_rng(7)
    bits = synth.f32_to_bf16((rng.standard_normal((64, 128)) * 3).astype(np.float32))
    w8 = synth.Workload("kv8_pin", 1, 4, 4, 4, 1, kv_dtype="fp8")
    got = oracle.kv_values_bf16(w8, bits)
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    ref = t.to(torch.float8_e4m3fn).to(torch.float32).numpy()
    assert np.array_equal((got.astype(np.uint32) << 16).view(np.float32), ref)
    assert oracle.kv_values_bf16(synth.Workload("kv_pin", 1, 4, 4, 4, 1), bits) is bits
