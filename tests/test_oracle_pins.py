"""The fp64 oracle against library routines, closed forms and invariants."""

import numpy as np
import pytest

import oracle
import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def test_rejects_malformed_arguments():
    from workloads import make_batch
    b = make_batch([3], [3], 4, 2, 16, seed=1)
    with pytest.raises(ValueError):  # Hq not a multiple of Hkv
        oracle.ragged_attention(b.q, b.k.repeat(1, 2, 1)[:, :3].contiguous(),
                                b.v.repeat(1, 2, 1)[:, :3].contiguous(), b.q_indptr,
                                b.kv_indptr, 4, 3, True, 0.1)
    with pytest.raises(ValueError):  # decreasing offsets
        oracle.ragged_attention(b.q, b.k, b.v, [0, 3, 2], [0, 3, 3], 4, 2, True, 0.1)


def test_thread_count_does_not_change_bits():
    from workloads import make_batch
    b = make_batch([40, 7], [64, 7], 4, 2, 32, seed=2)
    n0 = oracle.num_threads()
    try:
        oracle.set_num_threads(1)
        o1, l1 = oracle.ragged_attention(b.q, b.k, b.v, b.q_indptr, b.kv_indptr, 4, 2, True, 0.2)
        oracle.set_num_threads(max(2, n0))
        o2, l2 = oracle.ragged_attention(b.q, b.k, b.v, b.q_indptr, b.kv_indptr, 4, 2, True, 0.2)
    finally:
        oracle.set_num_threads(n0)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
