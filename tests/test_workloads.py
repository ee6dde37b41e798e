"""The seeded workloads, and one GPU's share of a column split (CPU only)."""
import pytest
import torch

import workloads


def test_shards_are_column_splits_of_the_two_large_workloads():
    got = {(w.M, w.N, w.K, w.dist, w.scale, w.seed) for w in workloads.SHARDS}
    want = set()
    for base in (workloads.SQUARE_4096, workloads.SKINNY):
        for ways in (2, 4, 8):
            want.add((base.M, base.N // ways, base.K, base.dist, base.scale, base.seed))
    assert got == want
    for w in workloads.SHARDS:
        assert workloads.BY_NAME[w.name] is w
        assert f"_{w.M}x{w.N}x{w.K}_" in w.name and "_nsplit" in w.name
    # the five workloads stay the five
    assert len(workloads.ALL) == 5 and not set(workloads.ALL) & set(workloads.SHARDS)


def test_shard_counts_scale_with_the_split():
    base = workloads.SQUARE_4096
    for ways in (1, 2, 4, 8):
        s = workloads.n_shard(base, ways)
        assert s.flops * ways == base.flops
        # A is replicated: each shard still reads all of it
        assert s.min_bytes == 2 * (base.M * base.K + base.K * base.N // ways + base.M * base.N // ways)


def test_shard_rejects_uneven_split():
    with pytest.raises(ValueError):
        workloads.n_shard(workloads.RAGGED, 3)
    with pytest.raises(ValueError):
        workloads.n_shard(workloads.SQUARE_256, 0)


def test_shard_draws_the_same_a_as_the_full_problem():
    # A is drawn first from the same seed with the same shape, so every GPU's
    # replica of A equals the unsplit problem's A
    base = workloads.Workload("w_64x64x32_normal", 64, 64, 32, "normal", 1.0, 7)
    a_full, b_full = workloads.workload_inputs(base)
    a_shard, b_shard = workloads.workload_inputs(workloads.n_shard(base, 4))
    assert torch.equal(a_full, a_shard)
    assert b_shard.shape == (32, 16)


def test_input_distribution_ablation():
    w = workloads.with_dist(workloads.SQUARE_4096, "ones")
    assert (w.M, w.N, w.K, w.seed) == (4096, 4096, 4096, 0) and w.dist == "ones"
    assert w.name.endswith("_inputs-ones") and w.name not in workloads.BY_NAME
    assert workloads.with_dist(workloads.SQUARE_4096, "normal") is workloads.SQUARE_4096
    a, b = workloads.make_inputs(8, 4, 16, "ones")
    assert a.shape == (8, 16) and b.shape == (16, 4)
    assert torch.all(a == 1) and torch.all(b == 1) and a.dtype == torch.float16
    small = workloads.with_dist(workloads.SKINNY, "intsmall")
    a, b = workloads.workload_inputs(workloads.Workload("t", 8, 8, 8, small.dist, small.scale))
    assert set(torch.unique(torch.cat([a.flatten(), b.flatten()])).tolist()) <= {-2.0, -1.0, 0.0, 1.0, 2.0}
