"""pagedkv_check_tables (the host validation that PAGEDKV_DEBUG=1 runs before
every launch) through the host-only entry points, so that the sanitizer build
of the host code runs these too."""
import numpy as np
import pytest

import paged_kv_cache_193_amd as pkv


def _good():
    bt = np.array([[3, 1, 7, -1], [0, 2, -1, -1]], dtype=np.int32)   # -1 past the context
    cl = np.array([40, 17], dtype=np.int32)                           # 3 and 2 blocks used
    return bt, cl


def test_accepts_valid_tables():
    bt, cl = _good()
    pkv.check_tables(bt, cl, pkv.CHECK_READ, num_blocks=8)
    pkv.check_tables(bt, cl, pkv.CHECK_APPEND, num_blocks=8)                  # one new token each
    pkv.check_tables(bt, cl, pkv.CHECK_APPEND, np.array([0, 5, 9], np.int32), num_blocks=8)
    pkv.check_tables(bt, cl, pkv.CHECK_PREFILL, np.array([0, 40, 57], np.int32), num_blocks=8)
    pkv.check_tables(bt[:0], cl[:0], pkv.CHECK_READ, num_blocks=8)            # empty batch
    bt[0, 3] = 12345            # entries past the context are never read
    pkv.check_tables(bt, cl, pkv.CHECK_READ, num_blocks=8)


@pytest.mark.parametrize("where,value,match", [
    ((0, 2), 8, "physical block 8 outside"),
    ((1, 0), -1, "physical block -1 outside"),
])
def test_rejects_block_ids_outside_the_pool(where, value, match):
    bt, cl = _good()
    bt[where] = value
    with pytest.raises(pkv.PagedKVError, match=match) as e:
        pkv.check_tables(bt, cl, pkv.CHECK_READ, num_blocks=8)
    assert e.value.code == pkv.PKV_ERR_INVALID_ARG


@pytest.mark.parametrize("b,value", [(0, 65), (1, -2)])
def test_rejects_lengths_beyond_the_table(b, value):
    bt, cl = _good()
    cl[b] = value
    with pytest.raises(pkv.PagedKVError, match=f"context length {value} outside"):
        pkv.check_tables(bt, cl, pkv.CHECK_READ, num_blocks=8)


def test_rejects_inconsistent_counts():
    bt, cl = _good()
    with pytest.raises(pkv.PagedKVError, match="appends 18 tokens"):
        pkv.check_tables(bt, cl, pkv.CHECK_APPEND, np.array([0, 1, 19], np.int32), num_blocks=8)
    with pytest.raises(pkv.PagedKVError, match="41 query tokens but only 40"):
        pkv.check_tables(bt, cl, pkv.CHECK_PREFILL, np.array([0, 41, 42], np.int32), num_blocks=8)
    with pytest.raises(pkv.PagedKVError, match="decrease"):
        pkv.check_tables(bt, cl, pkv.CHECK_PREFILL, np.array([0, 5, 3], np.int32), num_blocks=8,
                         T=3)
    with pytest.raises(pkv.PagedKVError, match="end at"):
        pkv.check_tables(bt, cl, pkv.CHECK_PREFILL, np.array([0, 5, 9], np.int32), num_blocks=8,
                         T=10)
    with pytest.raises(pkv.PagedKVError, match="start at"):
        pkv.check_tables(bt, cl, pkv.CHECK_APPEND, np.array([1, 5, 9], np.int32), num_blocks=8,
                         T=9)
    with pytest.raises(pkv.PagedKVError, match="T \\(3\\) == B"):
        pkv.check_tables(bt, cl, pkv.CHECK_APPEND, num_blocks=8, T=3)
