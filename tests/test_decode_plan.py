"""The decode launch plan (pa_decode_plan in include/pa.h) on the CPU.

pa_decode sizes its partition kernel's LDS on the host: the batch's schedule,
the table slices, query blocks and wave partials, then as many result-ring
slots as fit. A request larger than a compute unit's LDS once aborted a
queue on the GPU, so every shape the library accepts must fit and every
other one must be refused with PA_ERR_UNSUPPORTED before anything is
launched. pa_decode_plan is the same host computation pa_decode runs, with
the device's LDS sizes passed in, so the sweep here needs no GPU.

The expected sizes are the kernels' LDS layouts restated from their
documented regions (schedule arrays, table slices, query blocks, partials,
ring slots), not computed by the library.
"""

import ctypes

import pytest

LDS = 163840  # MI355X: bytes of LDS per compute unit, and per workgroup
GRANULE = 1024
F32, BF16, F16 = 0, 1, 2
VALU, MFMA, WAVE, STREAM = 0, 1, 2, 3
WAVES = 4
WAVE_SLICE = 128   # table entries per wave of the one-item-per-wave kernel
TABLE_SLICE = 512  # table entries of a workgroup item
MAX_RING = 32


def _lib():
    from paged_kv_cache_165_amd import _lib as L
    import os
    if not os.path.exists(L.LIB_PATH):
        pytest.skip("libpa.so not built (run __graft_entry__.build())")
    return L.load(), L


def _alloc(n):
    return (n + GRANULE - 1) // GRANULE * GRANULE


def _sched_ints(s):
    # fullpre[S + 1] | plist[S] | lens[S] (each padded to 4 ints) | 256 size
    # classes | the build's per-wave totals and per-wave class counts
    return ((s + 4) & ~3) + 2 * ((s + 3) & ~3) + 256 + WAVES + WAVES * 256


def _slot_bytes(g, d, stream=False):
    # o[G][D] | m[G] | l[G] | four ints of metadata, padded to 16 bytes
    return ((g * d + 2 * g + 4 + 3) & ~3) * 4


def _stream_sched_ints(s):
    # lens[S] | cs[S + 1] (each padded to 4 ints) | per-wave scan totals
    return ((s + 3) & ~3) + ((s + 4) & ~3) + WAVES


def _fixed_bytes(kernel, s, d, g):
    partials = WAVES * g * (d + 4) * 4   # per wave and head: D sums, max, sum (+2 pad)
    if kernel == VALU:
        return (_sched_ints(s) + TABLE_SLICE) * 4 + partials
    qw = (g * d // 2 + 3) & ~3           # 32-bit words of an item's query block
    if kernel == STREAM:
        return (_stream_sched_ints(s) + WAVES * WAVE_SLICE) * 4 + WAVES * qw * 4
    if kernel == MFMA:
        return (_sched_ints(s) + 2 * TABLE_SLICE) * 4 + 2 * qw * 4 + (2 if g * d <= 1024 else 1) * partials
    return (_sched_ints(s) + WAVES * WAVE_SLICE) * 4 + WAVES * qw * 4


def _expected(dt, d, g, s, part_blocks, max_wg, block_size=16, kv_heads=2, max_ctx=8192):
    """Kernel, LDS bytes, ring slots and residency the plan must give, or
    None when nothing fits."""
    mfma = dt != F32 and g >= 2
    # the stream split: 16-bit elements, any group and block size
    stream = (dt != F32 and part_blocks <= WAVE_SLICE and
              s * kv_heads * (4 * max(1, -(-max_ctx // 16)) + 3) < 2 ** 31 - 1)
    if stream:   # the stream split's records differ: no other kernel stands in
        cands = [STREAM]
    else:
        cands = ([WAVE] if mfma and part_blocks <= WAVE_SLICE else []) + ([MFMA] if mfma else [VALU])
    for k in cands:
        cap = min(1, max_wg) if k != VALU else max_wg
        mult = WAVES if k in (WAVE, STREAM) else 1
        fixed, slot = _fixed_bytes(k, s, d, g), _slot_bytes(g, d, k == STREAM)
        if _alloc(fixed + slot) > LDS:
            continue
        share = LDS // cap
        n = 1
        while n < MAX_RING and _alloc(fixed + (n + 1) * slot) <= share:
            n += 1
        n = n // mult * mult
        if n < 1:
            continue
        lds = fixed + n * slot
        return k, lds, n, min(cap, LDS // _alloc(lds))
    return None


SEQS = [0, 1, 7, 256, 1000, 2048, 4096, 6000, 7000, 8192]


@pytest.mark.parametrize("dt", [F32, BF16, F16])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("g", [1, 2, 4, 8, 16])
def test_every_accepted_plan_fits_and_the_rest_is_refused(dt, d, g):
    lib, L = _lib()
    plan = L.DecodePlan()
    refused = 0
    for part in (512, 2048, 4096, 8192):       # 32 .. 512 blocks of 16 tokens
        for max_wg in (1, 2, 3, 4):
            last_ok = True
            for s in SEQS:
                st = lib.pa_decode_plan(s, 2 * g, 2, d, 8192, 16, part, dt, LDS, LDS, max_wg, ctypes.byref(plan))
                if dt == F32 and g == 16:      # no float32 kernel for 16 heads per KV head
                    assert st == L.PA_ERR_UNSUPPORTED
                    continue
                exp = _expected(dt, d, g, s, part // 16, max_wg)
                if exp is None:
                    assert st == L.PA_ERR_UNSUPPORTED, (s, part, max_wg)
                    assert b"LDS" in lib.pa_last_error()
                    refused += 1
                    last_ok = False
                    continue
                assert st == L.PA_OK, (s, part, max_wg, lib.pa_last_error())
                assert last_ok, f"{s} sequences fit after a smaller batch did not"
                k, lds, ring, resident = exp
                assert (plan.kernel, plan.lds_bytes, plan.ring_slots, plan.workgroups_per_cu) == (k, lds, ring,
                                                                                                resident)
                assert plan.partition_size == part
                # the request fits one workgroup, and the resident ones fit the compute unit
                assert _alloc(plan.lds_bytes) <= LDS
                assert plan.workgroups_per_cu >= 1
                assert plan.workgroups_per_cu * _alloc(plan.lds_bytes) <= LDS
                if plan.kernel in (WAVE, STREAM):
                    assert plan.ring_slots % WAVES == 0
                if plan.kernel != VALU:
                    assert plan.workgroups_per_cu == 1
    if (dt, d, g) == (BF16, 256, 16):
        assert refused > 0  # the largest batches of the largest shape do not fit


def test_block_size_and_cost_bound_choose_the_kernel():
    lib, L = _lib()
    plan = L.DecodePlan()
    for bs, part, kernel in [(16, 2048, STREAM), (32, 4096, STREAM), (8, 1024, STREAM), (4, 512, STREAM),
                             (16, 4096, MFMA)]:  # 256 blocks: more than a wave's table slice
        assert lib.pa_decode_plan(64, 32, 8, 128, 8192, bs, part, BF16, LDS, LDS, 1, ctypes.byref(plan)) == 0
        assert plan.kernel == kernel, (bs, part)
    # stream cost positions are int32: a batch whose cost could pass 2^31 keeps the wave kernel
    assert lib.pa_decode_plan(8192, 64, 8, 128, 2 ** 20, 16, 2048, BF16, LDS, LDS, 1, ctypes.byref(plan)) == 0
    assert plan.kernel == WAVE


def test_plan_follows_the_default_partition_and_the_device_lds():
    lib, L = _lib()
    plan = L.DecodePlan()
    # the GQA batch-256 shape: 2048-token partitions, the stream split
    assert lib.pa_decode_plan(256, 32, 8, 128, 8192, 16, 0, BF16, LDS, LDS, 1, ctypes.byref(plan)) == 0
    assert plan.kernel == STREAM and plan.partition_size == 2048
    # blocks of 8 tokens: the stream split at 1024-token partitions
    assert lib.pa_decode_plan(256, 32, 8, 128, 8192, 8, 0, BF16, LDS, LDS, 1, ctypes.byref(plan)) == 0
    assert plan.kernel == STREAM and plan.partition_size == 1024
    # a smaller LDS holds fewer ring slots, and a too small one refuses
    assert lib.pa_decode_plan(256, 32, 8, 128, 8192, 16, 0, BF16, 65536, 65536, 1, ctypes.byref(plan)) == 0
    small = plan.ring_slots
    assert lib.pa_decode_plan(256, 32, 8, 128, 8192, 16, 0, BF16, LDS, LDS, 1, ctypes.byref(plan)) == 0
    assert plan.ring_slots > small
    assert lib.pa_decode_plan(4096, 32, 8, 128, 8192, 16, 0, BF16, 16384, 16384, 1,
                              ctypes.byref(plan)) == L.PA_ERR_UNSUPPORTED
    # partitions over 128 blocks run one item per workgroup
    assert lib.pa_decode_plan(64, 32, 8, 128, 8192, 16, 4096, BF16, LDS, LDS, 1, ctypes.byref(plan)) == 0
    assert plan.kernel == MFMA
    # one query head per KV head: the stream split (here at 2048 and 1024
    # tokens), the VALU kernel with partitions over 128 blocks and for float32
    assert lib.pa_decode_plan(64, 32, 32, 128, 4096, 16, 0, BF16, LDS, LDS, 2, ctypes.byref(plan)) == 0
    assert plan.kernel == STREAM and plan.partition_size == 2048 and plan.workgroups_per_cu == 1
    assert lib.pa_decode_plan(64, 32, 32, 128, 4096, 8, 0, BF16, LDS, LDS, 2, ctypes.byref(plan)) == 0
    assert plan.kernel == STREAM and plan.partition_size == 1024
    assert lib.pa_decode_plan(64, 32, 32, 128, 4096, 16, 4096, BF16, LDS, LDS, 2, ctypes.byref(plan)) == 0
    assert plan.kernel == VALU and plan.workgroups_per_cu == 2
    assert lib.pa_decode_plan(64, 32, 32, 128, 4096, 16, 0, F32, LDS, LDS, 2, ctypes.byref(plan)) == 0
    assert plan.kernel == VALU and plan.partition_size == 4096


def test_plan_rejects_bad_arguments():
    lib, L = _lib()
    plan = L.DecodePlan()
    assert lib.pa_decode_plan(4, 8, 8, 128, 100, 16, 0, BF16, LDS, LDS, 1, None) == L.PA_ERR_INVALID_ARG
    for bad in [(4, 8, 8, 128, 100, 16, 0, BF16, 0, LDS, 1), (4, 8, 8, 128, 100, 16, 0, BF16, LDS, 0, 1),
                (4, 8, 8, 128, 100, 16, 0, BF16, LDS, LDS, 0), (4, 8, 3, 128, 100, 16, 0, BF16, LDS, LDS, 1),
                (-1, 8, 8, 128, 100, 16, 0, BF16, LDS, LDS, 1), (4, 8, 8, 128, 100, 16, 24, BF16, LDS, LDS, 1)]:
        assert lib.pa_decode_plan(*bad, ctypes.byref(plan)) == L.PA_ERR_INVALID_ARG, bad
    assert lib.pa_decode_plan(4, 8, 8, 96, 100, 16, 0, BF16, LDS, LDS, 1, ctypes.byref(plan)) == \
        L.PA_ERR_UNSUPPORTED
    assert lib.pa_decode_plan(8193, 8, 8, 128, 100, 16, 0, BF16, LDS, LDS, 1, ctypes.byref(plan)) == \
        L.PA_ERR_UNSUPPORTED
