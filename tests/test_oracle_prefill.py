"""Pins of the oracle's paged prefill (multi-token query) attention: it
reduces to paged decode for one new token per sequence, a whole prompt equals
float64 causal scaled_dot_product_attention (library routine), small cases
equal a pure-Python scalar loop, the last new token equals a decode over the
full context, and planted mistakes in the causal bound or the positions are
each caught by at least one pin."""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import F32
from test_oracle import vstore


def _prefill(q, kc, vc, tables, lens, qstart, scale, bs, dtype=F32):
    """The pins pass logical V; the oracle reads the storage layout."""
    return oracle.paged_prefill(q, kc, vstore(vc), tables, lens, qstart, scale, bs, dtype)


def _case(seed, lens, news, hq, hkv, d, bs, pool):
    rng = np.random.default_rng(seed)
    need = [-(-L // bs) for L in lens]
    tables = np.zeros((len(lens), max(max(need), 1)), np.int64)
    perm = rng.permutation(pool)
    k = 0
    for i, n in enumerate(need):
        tables[i, :n] = perm[k:k + n]
        k += n
    kc = rng.standard_normal((pool, hkv, bs, d)).astype(np.float32)
    vc = rng.standard_normal((pool, hkv, bs, d)).astype(np.float32)
    qstart = np.concatenate([[0], np.cumsum(news)]).astype(np.int64)
    q = rng.standard_normal((int(qstart[-1]), hq, d)).astype(np.float32)
    return q, kc, vc, tables, np.array(lens), qstart


def pin_one_new_token_is_decode(prefill):
    lens = [1, 17, 64, 100]
    q, kc, vc, tables, lens_a, qs = _case(1, lens, [1, 1, 1, 1], 8, 2, 16, 16, 20)
    out = prefill(q, kc, vc, tables, lens_a, qs, 0.3, 16)
    ref = oracle.paged_decode(q, kc, vstore(vc), tables, lens_a, 0.3, 16, F32)
    assert np.array_equal(out, ref)


def pin_whole_prompt_is_causal_sdpa(prefill):
    """Contiguous blocks, every token new: torch's float64 causal attention
    with the KV heads repeated per group."""
    bs, hq, hkv, d, L = 8, 4, 2, 16, 37
    q, kc, vc, _, _, _ = _case(2, [L], [L], hq, hkv, d, bs, 5)
    out = prefill(q, kc, vc, np.arange(5)[None, :], np.array([L]), np.array([0, L]), 0.2, bs)
    kk = torch.from_numpy(kc.astype(np.float64)).permute(1, 0, 2, 3).reshape(hkv, -1, d)[:, :L]
    vv = torch.from_numpy(vc.astype(np.float64)).permute(1, 0, 2, 3).reshape(hkv, -1, d)[:, :L]
    kk = kk.repeat_interleave(hq // hkv, dim=0)[None]
    vv = vv.repeat_interleave(hq // hkv, dim=0)[None]
    qq = torch.from_numpy(q.astype(np.float64)).permute(1, 0, 2)[None]  # [1, hq, L, d]
    ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, is_causal=True, scale=0.2)
    np.testing.assert_allclose(out, ref[0].permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def _brute(q, kc, vc, tables, lens, qs, scale, bs):
    out = np.zeros(q.shape)
    hq, d = q.shape[1], q.shape[2]
    g = hq // kc.shape[1]
    for s in range(len(lens)):
        L, m = int(lens[s]), int(qs[s + 1] - qs[s])
        for j in range(m):
            p = L - m + j
            for h in range(hq):
                xs = []
                for t in range(p + 1):
                    pid, off = int(tables[s][t // bs]), t % bs
                    xs.append(scale * sum(float(q[qs[s] + j, h, e]) * float(kc[pid, h // g, off, e]) for e in range(d)))
                mx = max(xs)
                w = [math.exp(x - mx) for x in xs]
                for e in range(d):
                    acc = sum(w[t] * float(vc[int(tables[s][t // bs]), h // g, t % bs, e]) for t in range(p + 1))
                    out[qs[s] + j, h, e] = acc / sum(w)
    return out


def pin_brute_force(prefill):
    lens, news = [5, 9, 16], [5, 3, 2]
    q, kc, vc, tables, lens_a, qs = _case(3, lens, news, 4, 2, 4, 4, 12)
    out = prefill(q, kc, vc, tables, lens_a, qs, 0.5, 4)
    np.testing.assert_allclose(out, _brute(q, kc, vc, tables, lens_a, qs, 0.5, 4), rtol=0, atol=1e-12)


def pin_last_token_is_full_decode(prefill):
    lens, news = [30, 47], [6, 47]
    q, kc, vc, tables, lens_a, qs = _case(4, lens, news, 4, 4, 8, 8, 16)
    out = prefill(q, kc, vc, tables, lens_a, qs, 0.4, 8)
    last = np.array([qs[1] - 1, qs[2] - 1])
    ref = oracle.paged_decode(q[last], kc, vstore(vc), tables, lens_a, 0.4, 8, F32)
    assert np.array_equal(out[last], ref)


PINS = [pin_one_new_token_is_decode, pin_whole_prompt_is_causal_sdpa, pin_brute_force,
        pin_last_token_is_full_decode]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_prefill_pins(pin):
    pin(_prefill)


def _mutant(kind):
    def prefill(q, kc, vc, tables, lens, qs, scale, bs, dtype=F32):
        out = np.zeros(q.shape)
        g = q.shape[1] // kc.shape[1]
        for s in range(len(lens)):
            L, m = int(lens[s]), int(qs[s + 1] - qs[s])
            t = np.arange(L)
            K = kc[tables[s][t // bs], :, t % bs, :].astype(np.float64)
            V = vc[tables[s][t // bs], :, t % bs, :].astype(np.float64)
            for j in range(m):
                p = L - m + j
                if kind == "exclusive_bound":
                    p = p - 1
                elif kind == "positions_from_start":
                    p = j
                elif kind == "no_mask":
                    p = L - 1
                if p < 0:
                    continue
                for h in range(q.shape[1]):
                    x = scale * (K[:p + 1, h // g] @ q[qs[s] + j, h].astype(np.float64))
                    w = np.exp(x - x.max())
                    out[qs[s] + j, h] = (w @ V[:p + 1, h // g]) / w.sum()
        return out
    return prefill


MUTANTS = ["exclusive_bound", "positions_from_start", "no_mask"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_prefill_pins_catch_planted_mistake(kind):
    bad = _mutant(kind)
    caught = []
    for pin in PINS:
        try:
            pin(bad)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches mutant {kind}"


def test_unmutated_prefill_copy_passes_all_pins():
    good = _mutant("none")
    for pin in PINS:
        pin(good)


def test_prefill_rejects_bad_query_start():
    q, kc, vc, tables, lens_a, qs = _case(5, [4], [4], 2, 2, 4, 4, 2)
    with pytest.raises(ValueError):
        _prefill(q, kc, vc, tables, lens_a, np.array([0, 5]), 0.5, 4)
    with pytest.raises(ValueError):
        _prefill(q, kc, vc, tables, np.array([3]), qs, 0.5, 4)
