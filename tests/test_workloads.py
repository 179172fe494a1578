"""CPU checks of the seeded input generator's skew mixes and structure builder
(input generation only; the generator holds none of the method's arithmetic)."""

import numpy as np
import pytest

import workloads


@pytest.mark.parametrize("mix", workloads.SKEW_MIXES)
@pytest.mark.parametrize("batch", [1, 4, 16, 64, 128])
def test_skew_lengths_sum_and_floor(mix, batch):
    lens = workloads.skew_lengths(mix, batch)
    assert lens.shape == (batch,) and lens.dtype == np.int32
    assert int(lens.sum()) == workloads.SKEW_TOTAL
    assert int(lens.min()) >= 16
    assert np.array_equal(lens, workloads.skew_lengths(mix, batch))  # seeded


def test_skew_mix_shapes():
    u = workloads.skew_lengths("uniform", 64)
    assert u.max() - u.min() <= 1
    one = workloads.skew_lengths("one-long", 64)
    assert abs(int(one.max()) - workloads.SKEW_TOTAL // 2) <= 64 * 16  # about half (the floors aside)
    heavy = workloads.skew_lengths("heavy", 128)
    assert heavy.max() > 8 * np.median(heavy)  # a heavy tail


def test_structure_for_lengths_covers_every_key():
    lens = np.array([1, 17, 300, 16, 33], np.int32)
    st = workloads.structure_for_lengths(9, lens, block_size=16)
    tables, bs = st["block_tables"], st["block_size"]
    used = []
    for s, n in enumerate(lens):
        nb = -(-int(n) // bs)
        assert np.all(tables[s, :nb] >= 0) and np.all(tables[s, nb:] == -1)
        used.extend(tables[s, :nb].tolist())
    assert sorted(used) == list(range(st["num_blocks"]))  # each pool block owned once
    # this step's slot of each sequence is its last key
    for s, n in enumerate(lens):
        last = int(n) - 1
        assert st["slot_mapping"][s] == tables[s, last // bs] * bs + last % bs
    assert np.array_equal(st["cu_seqlens"], np.arange(6, dtype=np.int32))
