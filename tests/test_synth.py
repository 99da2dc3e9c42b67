"""The seeded input generator: definition, distribution, planting, and (on a
GPU) bit-equality of the device fill with the host generator."""
import numpy as np
import pytest

import synth


def test_splitmix_vectorised_matches_integer_form():
    rng = np.random.default_rng(5)
    xs = rng.integers(0, 2**63, size=200, dtype=np.uint64)
    v = synth._sm64_np(xs)
    for x, y in zip(xs.tolist(), v.tolist()):
        assert synth._sm64_int(int(x)) == int(y)


def test_splitmix_published_sequence():
    """SplitMix64 seeded with 0: first output of Vigna's reference generator."""
    assert synth._sm64_int(0) == 0xE220A8397B1DCDAF


def test_bf16_round_to_nearest_even():
    cases = [
        (1.0, 0x3F80),
        (1.0 + 2**-8, 0x3F80),              # exact tie, round to even (down)
        (1.0 + 3 * 2**-8, 0x3F82),          # exact tie, round to even (up)
        (1.0 + 2**-8 + 2**-20, 0x3F81),     # above the tie
        (-2.5, 0xC020),
        (0.0, 0x0000),
        (-0.0, 0x8000),
    ]
    for x, bits in cases:
        assert int(synth.f32_to_bf16(np.float32(x)).reshape(-1)[0]) == bits, x


def test_normal_table_is_standard_normal():
    t = synth.bf16_to_f32(synth.normal_table()).astype(np.float64)
    assert abs(t.mean()) < 1e-3 and abs(t.std() - 1.0) < 2e-3
    assert np.all(np.diff(t) >= 0)                     # quantiles are monotone
    assert np.array_equal(t, -t[::-1])                 # symmetric
    assert abs(t.max() - 4.3249) < 0.02


def test_generated_values_and_ranges_agree():
    a = synth.gen_range(7, synth.T_Q, 1000, 5000)
    b = synth.gen_at(7, synth.T_Q, np.arange(1000, 6000))
    assert np.array_equal(a, b)
    x = synth.bf16_to_f32(synth.gen_range(7, synth.T_K, 0, 200000)).astype(np.float64)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01
    assert not np.array_equal(synth.gen_range(7, synth.T_K, 0, 64), synth.gen_range(7, synth.T_V, 0, 64))


def test_planting_raises_planted_blocks():
    w = synth.WORKLOADS["prefill_4k"]
    p = synth.plant_spec(w)
    assert len(p.blocks) == 1 and len(set(p.blocks[0])) == 3
    assert abs(np.linalg.norm(p.vec_k[0].astype(np.float64)) - w.plant_alpha) < 1e-4
    ik = synth.host_ik(w, 0, 0, w.n_kv, p)
    raw = synth.gen_range(w.seed, synth.T_IK, 0, w.n_kv * w.index_dim).reshape(w.n_kv, w.index_dim)
    changed = np.any(ik != raw, axis=1)
    planted_rows = np.zeros(w.n_kv, bool)
    for t in p.blocks[0]:
        planted_rows[t * 128:(t + 1) * 128] = True
    assert not np.any(changed & ~planted_rows)
    # the planted direction is visible in the keys
    u = p.vec_k[0] / np.linalg.norm(p.vec_k[0])
    proj = synth.bf16_to_f32(ik) @ u
    assert proj[planted_rows].mean() > 12 and abs(proj[~planted_rows].mean()) < 0.2


def test_row_generators_agree_with_ranges():
    w = synth.WORKLOADS["prefill_32k"]
    rows = np.array([0, 5, 1000, 32767])
    a = synth.host_iq_rows(w, 0, rows)
    for n, r in enumerate(rows):
        assert np.array_equal(a[n], synth.host_iq(w, 0, int(r), int(r) + 1)[0])
    q = synth.host_q_rows(w, 0, rows)
    assert np.array_equal(q[2], synth.host_q(w, 0, 1000, 1001)[0])


@pytest.mark.gpu
def test_device_fill_matches_host():
    import torch
    w = synth.WORKLOADS["prefill_32k"].replace(n_q=4096, n_kv=4096)
    dev = synth.device_inputs(w)
    host = synth.host_all(w)
    for name in ("q", "k", "v", "iq", "ik"):
        d = dev[name].view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(d, host[name]), name


@pytest.mark.gpu
def test_device_fill_samples_at_large_offsets():
    """Sampled elements of a tensor larger than 2**32 elements."""
    import torch
    w = synth.WORKLOADS["decode_256k"].replace(batch=20)   # 5.4e9 elements
    nt = torch.from_numpy(synth.normal_table().view(np.int16).copy()).cuda()
    k = torch.empty(w.shapes()["k"], dtype=torch.bfloat16, device="cuda")
    synth.device_fill(w, "k", k, nt_dev=nt)
    torch.cuda.synchronize()
    flat = k.view(-1)
    idx = np.concatenate([np.arange(0, 16), np.random.default_rng(0).integers(0, flat.numel(), 2000),
                          np.arange(flat.numel() - 16, flat.numel())])
    got = flat[torch.from_numpy(idx).cuda()].view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, synth.gen_at(w.seed, synth.T_K, idx))


def test_v_outlier_channels_are_exact_power_of_two_multiples():
    """v_outlier_shift multiplies V's outlier channels by 2**shift exactly
    (exponent field), leaves zeros and every other channel and tensor alone."""
    w = synth.Workload("v_outlier", 1, 512, 512, 4, 2, seed=77, v_outlier_shift=3)
    base = w.replace(v_outlier_shift=0)
    a, b = synth.host_kv(w, "v", 0, 1, 0, 512), synth.host_kv(base, "v", 0, 1, 0, 512)
    f = lambda x: (x.astype(np.uint32) << 16).view(np.float32)
    others = [c for c in range(w.head_dim) if c not in synth.V_OUTLIER_DIMS]
    assert np.array_equal(a[:, others], b[:, others])
    for c in synth.V_OUTLIER_DIMS:
        assert np.array_equal(f(a[:, c]), f(b[:, c]) * 8.0)
    assert np.array_equal(synth.host_kv(w, "k", 0, 1, 0, 512), synth.host_kv(base, "k", 0, 1, 0, 512))
    z = np.zeros((2, w.head_dim), np.uint16)
    assert np.array_equal(synth._outlier_bits(z, 3), z)
