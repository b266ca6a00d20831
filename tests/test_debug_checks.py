"""The opt-in precondition checks of the binding (PA_DEBUG=1) on host arrays.

The kernels clamp bad indices instead of faulting and cannot report a broken
precondition; these host checks (the debug consistency check of the cf-1.com
blog, 4.3) reject each kind before a call is made. No GPU."""

import numpy as np
import pytest

import paged_kv_cache_165_amd as pa


def test_slot_mapping_checks():
    pa.check_slot_mapping(np.array([-1, 0, 5, 63, -1], np.int32), num_blocks=16, block_size=4)
    pa.check_slot_mapping(np.zeros(0, np.int32), 16, 4)
    with pytest.raises(ValueError, match="more than once"):
        pa.check_slot_mapping(np.array([3, 7, 3], np.int32), 16, 4)
    with pytest.raises(ValueError, match="outside"):
        pa.check_slot_mapping(np.array([64], np.int32), 16, 4)     # one past the pool
    with pytest.raises(ValueError, match="outside"):
        pa.check_slot_mapping(np.array([-2], np.int32), 16, 4)


def test_copy_pair_checks():
    pa.check_copy_pairs(np.array([[1, 2], [1, 3], [4, 5]], np.int32), num_blocks=8)  # one source, two copies
    with pytest.raises(ValueError, match="more than once"):
        pa.check_copy_pairs(np.array([[1, 2], [3, 2]], np.int32), 8)
    with pytest.raises(ValueError, match="both a copy source and a copy destination"):
        pa.check_copy_pairs(np.array([[1, 2], [2, 3]], np.int32), 8)
    with pytest.raises(ValueError, match="outside"):
        pa.check_copy_pairs(np.array([[1, 8]], np.int32), 8)
    with pytest.raises(ValueError, match="outside"):
        pa.check_copy_pairs(np.array([[-1, 2]], np.int32), 8)


def test_decode_input_checks():
    tables = np.array([[5, 1, 7], [2, 9, 9]], np.int32)   # row 1 reads one entry; its padding is never read
    pa.check_decode_inputs(tables, np.array([10, 3], np.int32), num_blocks=8, block_size=4, max_context_len=12)
    with pytest.raises(ValueError, match="outside"):
        pa.check_decode_inputs(tables, np.array([10, 5], np.int32), 8, 4, 12)   # now reads block 9
    with pytest.raises(ValueError, match="context_lens"):
        pa.check_decode_inputs(tables, np.array([13, 3], np.int32), 8, 4, 12)
    with pytest.raises(ValueError, match="context_lens"):
        pa.check_decode_inputs(tables, np.array([-1, 3], np.int32), 8, 4, 12)
    with pytest.raises(ValueError, match="more table entries"):
        pa.check_decode_inputs(tables, np.array([13, 3], np.int32), 8, 4, 16)


def test_debug_switch(monkeypatch):
    monkeypatch.delenv("PA_DEBUG", raising=False)
    assert not pa.debug_enabled()
    monkeypatch.setenv("PA_DEBUG", "1")
    assert pa.debug_enabled()
