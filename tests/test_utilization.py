"""The contiguous-versus-paged allocation simulator
(paged_kv_cache_165_amd.utilization), host only: the waste ratio and the
paged internal-fragmentation estimate of the aiqz.cc tutorial (section
显存收益分析) on closed-form cases, a one-request trace worked by hand, token
conservation, the preemption path, and the ordering the tutorial argues
(paged wastes less and runs more requests at once on the same cache)."""

import os

import numpy as np
import pytest


def _u():
    from paged_kv_cache_165_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libpa.so not built")
    from paged_kv_cache_165_amd import utilization
    return utilization


def test_static_waste_closed_forms():
    U = _u()
    r = U.static_waste([16, 32, 48, 160], 16, 256)
    assert r["paged_waste"] == 0.0                      # whole blocks: nothing wasted
    assert r["contiguous_waste"] == pytest.approx(1 - 256 / (4 * 256))
    r = U.static_waste([1, 17], 16, 64)                 # 1 block + 2 blocks, 18 used of 48
    assert r["paged_alloc_slots"] == 48 and r["paged_waste"] == pytest.approx(30 / 48)
    assert r["contiguous_waste"] == pytest.approx(1 - 18 / 128)
    with pytest.raises(ValueError):
        U.static_waste([300], 16, 256)


def test_half_a_block_per_request():
    """Lengths spread evenly over many block sizes: the measured paged waste
    is close to eta'_int = 1 / (2 N_blocks). Over integer lengths the empty
    tail of the last block is uniform on 0..B-1 slots, so its mean is
    (B - 1) / 2 slots rather than exactly half a block: the measured ratio is
    (B - 1) / B of the estimate."""
    U = _u()
    rng = np.random.default_rng(0)
    lens = rng.integers(16 * 100, 16 * 200, size=20000)
    r = U.static_waste(lens, 16, 16 * 200)
    assert r["paged_waste"] == pytest.approx(r["paged_internal_estimate"], rel=0.08)
    assert r["paged_waste"] == pytest.approx(r["paged_internal_estimate"] * 15 / 16, rel=0.02)


def test_one_request_by_hand():
    """Prompt 5, output 3, blocks of 4, max_new 8. Paged: 6, 7, 8 tokens in
    2 blocks (8 slots) over the three steps -> waste 2/8, 1/8, 0. Contiguous:
    13 reserved -> waste 7/13, 6/13, 5/13."""
    U = _u()
    tr = [U.Request(0, 5, 3)]
    p = U.simulate(tr, 64, "paged", block_size=4, max_new=8)
    assert p["steps"] == 3 and p["finished"] == 1 and p["generated_tokens"] == 3
    assert p["mean_waste"] == pytest.approx((2 / 8 + 1 / 8 + 0) / 3)
    c = U.simulate(tr, 64, "contiguous", block_size=4, max_new=8)
    assert c["mean_waste"] == pytest.approx((7 / 13 + 6 / 13 + 5 / 13) / 3)
    assert c["mean_running"] == p["mean_running"] == 1.0


def test_paged_runs_more_requests_and_wastes_less():
    U = _u()
    tr = U.make_trace(400, 3, arrivals_per_step=0.5)
    c = U.simulate(tr, 1 << 15, "contiguous")
    p = U.simulate(tr, 1 << 15, "paged")
    assert c["finished"] == p["finished"] == 400
    assert c["generated_tokens"] == sum(r.output for r in tr)
    # every token is generated once, plus those lost to preemption
    assert p["generated_tokens"] == sum(r.output for r in tr) + p["preempted_tokens"]
    assert p["mean_waste"] < 0.05 < 0.5 < c["mean_waste"]
    assert p["mean_running"] > 1.5 * c["mean_running"]
    assert p["steps"] < c["steps"]


def test_preemption_keeps_the_trace_moving():
    """A cache just large enough for a few long requests: requests must be
    preempted (by recomputation) and every one still finishes."""
    U = _u()
    tr = [U.Request(0, 64, 200) for _ in range(6)]
    p = U.simulate(tr, 16 * 40, "paged", block_size=16, max_new=256)
    assert p["finished"] == 6 and p["rejected"] == 0
    assert p["generated_tokens"] == 6 * 200 + p["preempted_tokens"]


def test_requests_that_never_fit_are_rejected():
    U = _u()
    tr = [U.Request(0, 100, 10), U.Request(1, 5000, 10)]
    c = U.simulate(tr, 2048, "contiguous", max_new=512)
    p = U.simulate(tr, 2048, "paged", max_new=512)
    assert c["rejected"] == p["rejected"] == 1 and c["finished"] == p["finished"] == 1
