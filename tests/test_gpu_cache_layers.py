"""Multi-layer cache write and block copy (pa_write_cache_layers,
pa_copy_blocks_layers through the C ABI) against the oracle, bit for bit:
every layer of a [L, ...] cache pair gets its own rows at the one slot
mapping, every layer's block is copied. NaN payloads in the new rows and
slots outside the pool (skipped) are included; the layered call must also
equal L single-layer calls on the layers' slices."""

import numpy as np
import pytest
import torch

import oracle
from harness import host_bits, log, raw_equal

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_165_amd as pa
    pa.library()


def _rand(g, shape, dtype):
    return torch.randn(*shape, generator=g, device=DEV).to(dtype)


CASES = [
    # dtype, layers, block size, head_dim, kv heads
    (torch.bfloat16, 1, 16, 128, 8),
    (torch.bfloat16, 3, 16, 128, 8),
    (torch.bfloat16, 8, 4, 64, 2),
    (torch.float16, 5, 64, 128, 4),
    (torch.float32, 4, 16, 64, 2),
    (torch.bfloat16, 2, 256, 256, 1),
]


@pytest.mark.parametrize("dt,nl,bs,d,hkv", CASES, ids=[f"{c[0]}-L{c[1]}-B{c[2]}-D{c[3]}" for c in CASES])
def test_write_layers_bit_exact(dt, nl, bs, d, hkv):
    import paged_kv_cache_165_amd as pa
    g = torch.Generator(device=DEV).manual_seed(nl * 1000 + bs)
    rng = np.random.default_rng(nl * 1000 + bs)
    nb = 24
    kc, vc = pa.alloc_cache_layers(nl, nb, hkv, bs, d, dt, device=DEV)
    kc.copy_(_rand(g, kc.shape, dt))
    vc.copy_(_rand(g, vc.shape, dt))
    n = 3 * bs + 5  # a run of consecutive slots, then scattered ones
    slots = np.concatenate([5 * bs + np.arange(2 * bs), rng.choice(np.arange(7 * bs, nb * bs), n - 2 * bs - 2,
                                                                    replace=False), [-1, nb * bs + 3]]).astype(np.int32)
    k, v = _rand(g, (nl, n, hkv, d), dt), _rand(g, (nl, n, hkv, d), dt)
    k[0, 1, 0, 0] = float("nan")
    kc_h, vc_h = host_bits(kc), host_bits(vc)
    log(f"[layers] write {dt} L={nl} B={bs} D={d} Hkv={hkv} tokens={n}")
    pa.write_cache_layers(k, v, kc, vc, torch.from_numpy(slots).to(DEV))
    torch.cuda.synchronize()
    keep = np.where((slots >= 0) & (slots < nb * bs), slots, -1)
    ref_k, ref_v = oracle.write_cache_layers(host_bits(k), host_bits(v), kc_h, vc_h, keep, bs)
    assert raw_equal(kc, ref_k) and raw_equal(vc, ref_v)


def test_write_layers_equals_single_layer_calls():
    import paged_kv_cache_165_amd as pa
    dt, nl, nb, hkv, bs, d = torch.bfloat16, 4, 16, 4, 16, 128
    g = torch.Generator(device=DEV).manual_seed(3)
    kc, vc = pa.alloc_cache_layers(nl, nb, hkv, bs, d, dt, device=DEV)
    kc.copy_(_rand(g, kc.shape, dt))
    vc.copy_(_rand(g, vc.shape, dt))
    kc2, vc2 = kc.clone(), vc.clone()
    slots = torch.arange(3, 3 + 40, dtype=torch.int32, device=DEV)
    k, v = _rand(g, (nl, 40, hkv, d), dt), _rand(g, (nl, 40, hkv, d), dt)
    pa.write_cache_layers(k, v, kc, vc, slots)
    for layer in range(nl):
        pa.write_cache(k[layer], v[layer], kc2[layer], vc2[layer], slots)
    torch.cuda.synchronize()
    assert torch.equal(kc.view(torch.int16), kc2.view(torch.int16))
    assert torch.equal(vc.view(torch.int16), vc2.view(torch.int16))


@pytest.mark.parametrize("dt,nl,bs,d,hkv", CASES, ids=[f"{c[0]}-L{c[1]}-B{c[2]}-D{c[3]}" for c in CASES])
def test_copy_layers_bit_exact(dt, nl, bs, d, hkv):
    import paged_kv_cache_165_amd as pa
    g = torch.Generator(device=DEV).manual_seed(nl * 100 + bs)
    nb = 20
    kc, vc = pa.alloc_cache_layers(nl, nb, hkv, bs, d, dt, device=DEV)
    kc.copy_(_rand(g, kc.shape, dt))
    vc.copy_(_rand(g, vc.shape, dt))
    pairs = np.array([[2, 11], [5, 0], [19, 7], [3, 12]], dtype=np.int32)
    kc_h, vc_h = host_bits(kc), host_bits(vc)
    log(f"[layers] copy {dt} L={nl} B={bs} D={d} Hkv={hkv} pairs={len(pairs)}")
    # an out-of-range pair is skipped
    dev_pairs = torch.from_numpy(np.concatenate([pairs, [[1, nb + 4]]]).astype(np.int32)).to(DEV)
    pa.copy_blocks_layers(kc, vc, dev_pairs)
    torch.cuda.synchronize()
    ref_k, ref_v = oracle.copy_blocks_layers(kc_h, vc_h, pairs)
    assert raw_equal(kc, ref_k) and raw_equal(vc, ref_v)
