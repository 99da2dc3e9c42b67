"""Compile-time checks of the HIP kernels (no GPU): no register spills to
scratch, and the hot kernels keep at least two waves per SIMD."""
import pytest

from block_sparse_long_qk_amd import build

HOT = ("k_index_scores", "k_attn_tiles", "k_index_small", "k_attn_rows", "k_block_topk", "k_attn_local_merge")


@pytest.fixture(scope="module")
def report():
    r = build.resource_report()
    assert r, "no kernel-resource-usage remarks from hipcc"
    return r


def test_no_scratch_spills(report):
    """No kernel uses scratch memory: neither the uniform-batch kernels nor
    the variable-length / paged instantiations spill a register to it."""
    def scratch(v):
        return max(v.get("ScratchSize [bytes/lane]", 0), 4 * v.get("VGPRs Spill", 0))
    bad = {k: v for k, v in report.items() if scratch(v)}
    assert not bad, bad


def test_hot_kernels_keep_two_waves(report):
    for name, v in report.items():
        if any(h in name for h in HOT) and "k_attn_rowsILi16E" not in name:  # the 16-head decode variant may run at one
            assert v.get("Occupancy [waves/SIMD]", 0) >= 2, (name, v)


def test_every_source_reports(report):
    names = " ".join(report)
    for k in HOT:
        assert k in names
