"""Pins of the oracle's multi-layer cache write and block copy: the write
probe of the lihaoran.work note's worked example (table [5, 1, 7], B = 4:
position 9 -> block 7, offset 1) and a copy probe hold in every layer with
layer-specific values, one layer equals the single-layer call, and two
planted mistakes (every layer written with layer 0's rows; only layer 0
copied) are caught."""

import numpy as np
import pytest

import oracle
from oracle import F32

B, NB, HKV, D, LAYERS = 4, 8, 2, 8, 3


def _caches(seed):
    rng = np.random.default_rng(seed)
    kc = rng.standard_normal((LAYERS, NB, HKV, B, D)).astype(np.float32)
    vc = rng.standard_normal((LAYERS, *oracle.v_cache_shape(NB, HKV, B, D))).astype(np.float32)
    return kc, vc


def _new(seed, n):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((LAYERS, n, HKV, D)).astype(np.float32),
            rng.standard_normal((LAYERS, n, HKV, D)).astype(np.float32))


def pin_write_probe(write):
    kc, vc = _caches(1)
    k, v = _new(2, 1)
    slot = 7 * B + 1  # position 9 of the table [5, 1, 7]
    assert oracle.translate([5, 1, 7], 9, B) == (7, 1)
    kc2, vc2 = write(k, v, kc, vc, [slot], B)
    for layer in range(LAYERS):
        assert np.array_equal(kc2[layer, 7, :, 1], k[layer, 0])
        assert np.array_equal(oracle.v_rows_at(vc2[layer], 7, 1, B), v[layer, 0])
    untouched = np.ones(kc.shape, bool)
    untouched[:, 7, :, 1] = False
    assert np.array_equal(kc2[untouched], kc[untouched])


def pin_one_layer_is_single_call(write):
    kc, vc = _caches(3)
    k, v = _new(4, 3)
    slots = [5, -1, 30]
    kc2, vc2 = write(k[:1], v[:1], kc[:1], vc[:1], slots, B)
    ref = oracle.write_cache(k[0], v[0], kc[0], vc[0], slots, B)
    assert np.array_equal(kc2[0], ref[0]) and np.array_equal(vc2[0], ref[1])


def pin_copy_probe(copy):
    kc, vc = _caches(5)
    kc2, vc2 = copy(kc, vc, [[2, 6], [3, 0]])
    for layer in range(LAYERS):
        assert np.array_equal(kc2[layer, 6], kc[layer, 2]) and np.array_equal(vc2[layer, 6], vc[layer, 2])
        assert np.array_equal(kc2[layer, 0], kc[layer, 3]) and np.array_equal(vc2[layer, 0], vc[layer, 3])
        keep = [b for b in range(NB) if b not in (6, 0)]
        assert np.array_equal(kc2[layer, keep], kc[layer, keep])


WRITE_PINS = [pin_write_probe, pin_one_layer_is_single_call]


@pytest.mark.parametrize("pin", WRITE_PINS, ids=[p.__name__ for p in WRITE_PINS])
def test_write_layers_pins(pin):
    pin(oracle.write_cache_layers)


def test_copy_layers_pin():
    pin_copy_probe(oracle.copy_blocks_layers)


def test_planted_mistakes_are_caught():
    def write_layer0_everywhere(k, v, kc, vc, slots, bs):
        return oracle.write_cache_layers(np.repeat(k[:1], len(k), 0), np.repeat(v[:1], len(v), 0), kc, vc, slots, bs)

    def copy_layer0_only(kc, vc, pairs):
        k0, v0 = oracle.copy_blocks(kc[0], vc[0], pairs)
        kc2, vc2 = kc.copy(), vc.copy()
        kc2[0], vc2[0] = k0, v0
        return kc2, vc2

    with pytest.raises(AssertionError):
        pin_write_probe(write_layer0_everywhere)
    with pytest.raises(AssertionError):
        pin_copy_probe(copy_layer0_only)


def test_layer_axis_required():
    kc, vc = _caches(6)
    k, v = _new(7, 1)
    with pytest.raises(ValueError):
        oracle.write_cache_layers(k[0], v[0], kc, vc, [1], B)
    with pytest.raises(ValueError):
        oracle.copy_blocks_layers(kc[0], vc[0], [[1, 2]])
