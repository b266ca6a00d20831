"""Pins for the CPU oracle: values the pages print, closed forms, invariants,
a textbook library routine and brute force. None of these re-types the
oracle's own formula. Runs without a GPU.

Each attention pin is written as a check that takes a decode function, so the
same pins are also run against deliberately broken copies of the oracle
(``MUTANTS`` below) to show that every plausible mistake is caught.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import BF16, F16, F32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# Block layout and address translation: values printed on the pages
# ---------------------------------------------------------------------------

def test_block_layout_printed_cases():
    g = _golden("block_layout.json")
    for c in g["layout_cases"]:
        assert oracle.block_layout(c["tokens"], c["block_size"]) == (c["blocks"], c["empty_slots"])
    # the page's printed line for 10 tokens
    assert "10 tokens: %s" % (oracle.block_layout(10, 4),) == g["printed_output"][0]


def test_block_layout_empty_slot_bound():
    g = _golden("block_layout.json")["empty_slot_bound"]
    for b in (g["block_size"], 16, 32):
        for n in range(g["tokens_from"], g["tokens_to_exclusive"]):
            blocks, unused = oracle.block_layout(n, b)
            assert blocks * b >= n and 0 <= unused < b
            # fewest blocks that hold n tokens: one fewer would not
            assert (blocks - 1) * b < n or n == 0
        assert oracle.block_layout(0, b) == (0, 0)


def test_block_layout_invalid():
    for c in _golden("block_layout.json")["invalid_inputs"]:
        with pytest.raises(ValueError):
            oracle.block_layout(c["tokens"], c["block_size"])


def test_quiz_q10_block_count():
    q = _golden("quiz_and_tables.json")["quiz_q10"]
    blocks, empty = oracle.block_layout(q["tokens"], q["block_size"])
    assert blocks == q["blocks"]
    assert q["block_size"] - empty == q["tokens_in_last_block"]


def test_translate_worked_example():
    c = _golden("block_layout.json")["translate_case"]
    pid, off = oracle.translate(c["block_table"], c["position"], c["block_size"])
    assert (pid, off) == (c["physical_block"], c["offset"])
    printed = "token %d -> physical block %d offset %d" % (c["position"], pid, off)
    assert printed == _golden("block_layout.json")["printed_output"][1]


def test_translate_block_table_sketch():
    c = _golden("quiz_and_tables.json")["block_table_example"]
    table = list(c["appended_physical_blocks"])
    # logical block 1 starts at token 1 * B for any block size
    for b in (1, 4, 16):
        assert oracle.translate(table, c["logical_block"] * b, b)[0] == c["physical_block"]


def test_bf16_decoding_of_known_patterns():
    pats = np.array([0x3F80, 0xC000, 0x3F81, 0x0000, 0x8000, 0x7F80, 0x4049], dtype=np.uint16)
    want = [1.0, -2.0, 1.0 + 2.0 ** -7, 0.0, -0.0, math.inf, 3.140625]
    got = oracle.to_float64(pats, BF16)
    assert list(got) == want
    assert math.copysign(1.0, got[4]) == -1.0


# ---------------------------------------------------------------------------
# Attention pins, written against a decode callable
# ---------------------------------------------------------------------------

def vstore(v_logical: np.ndarray) -> np.ndarray:
    """Logical V [NB, Hkv, B, D] -> the transposed tile storage
    [NB, Hkv, B // T, D, T] with T = min(B, 16) (test-side conversion)."""
    nb, hkv, bs, d = v_logical.shape
    t = min(bs, 16)
    return np.ascontiguousarray(v_logical.reshape(nb, hkv, bs // t, t, d).transpose(0, 1, 2, 4, 3))


def _decode(q, kc, vc, tables, lens, scale, bs, dtype=F32):
    """The pins pass logical V; the oracle reads the storage layout."""
    return oracle.paged_decode(q, kc, vstore(vc), tables, lens, scale, bs, dtype)


def pin_slot_id_probe(decode):
    """B = 4, ctx = 10, table [5, 1, 7], K == 0 and V holding its own slot id:
    the visited slots are 20..23, 4..7, 28, 29, whose mean is 165 / 10."""
    nb, hkv, bs, d = 8, 2, 4, 8
    kc = np.zeros((nb, hkv, bs, d), np.float32)
    vc = np.full((nb, hkv, bs, d), np.nan, np.float32)
    for pid in range(nb):
        for off in range(bs):
            vc[pid, :, off, :] = pid * bs + off
    vc[7, :, 2:, :] = np.nan  # empty tail slots of the last block are never read
    q = np.random.default_rng(0).standard_normal((1, 4, d)).astype(np.float32)
    out = decode(q, kc, vc, np.array([[5, 1, 7]]), np.array([10]), 0.3, bs)
    assert out.shape == (1, 4, d)
    assert np.all(out == 16.5), out


def pin_single_token(decode):
    """ctx = 1: the softmax weight is exactly 1, so the output is v_0."""
    rng = np.random.default_rng(1)
    nb, hkv, bs, d = 6, 2, 4, 16
    kc = rng.standard_normal((nb, hkv, bs, d)).astype(np.float32)
    vc = rng.standard_normal((nb, hkv, bs, d)).astype(np.float32)
    q = rng.standard_normal((1, 4, d)).astype(np.float32)
    out = decode(q, kc, vc, np.array([[3, 0]]), np.array([1]), 0.125, bs)
    for h in range(4):
        assert np.array_equal(out[0, h], vc[3, h // 2, 0, :].astype(np.float64))


def pin_zero_keys_give_mean(decode):
    """K == 0: every logit is 0, so the output is the mean of the visible V rows
    (rows past the context length hold NaN and must not be read)."""
    rng = np.random.default_rng(2)
    nb, hkv, bs, d = 10, 1, 4, 8
    kc = np.zeros((nb, hkv, bs, d), np.float32)
    vc = rng.standard_normal((nb, hkv, bs, d)).astype(np.float32)
    table = np.array([[9, 2, 4, 0]])
    vc[0, :, 3:, :] = np.nan  # ctx 15 -> last block holds 3 tokens
    q = rng.standard_normal((1, 1, d)).astype(np.float32)
    out = decode(q, kc, vc, table, np.array([15]), 1.0, bs)
    rows = [vc[table[0, t // bs], 0, t % bs, :].astype(np.float64) for t in range(15)]
    np.testing.assert_allclose(out[0, 0], np.mean(rows, axis=0), rtol=0, atol=1e-14)


def pin_gqa_head_mapping(decode):
    """Query head h reads KV head h // g: with 4 query heads on 2 KV heads,
    heads 0 and 1 see V == 0 and heads 2 and 3 see V == 1."""
    nb, hkv, bs, d = 2, 2, 4, 4
    kc = np.random.default_rng(3).standard_normal((nb, hkv, bs, d)).astype(np.float32)
    vc = np.zeros((nb, hkv, bs, d), np.float32)
    vc[:, 1] = 1.0
    q = np.random.default_rng(4).standard_normal((1, 4, d)).astype(np.float32)
    out = decode(q, kc, vc, np.array([[1, 0]]), np.array([7]), 0.5, bs)
    np.testing.assert_allclose(out[0, :, 0], [0.0, 0.0, 1.0, 1.0], atol=1e-15)


def pin_two_token_scale(decode):
    """Two keys k0 = 0 and k1 = c e_0, query e_0, scale s: the weights are
    1 / (1 + e^{sc}) and e^{sc} / (1 + e^{sc}) (softmax of [0, sc])."""
    bs, d = 4, 8
    kc = np.zeros((1, 1, bs, d), np.float32)
    vc = np.zeros((1, 1, bs, d), np.float32)
    c, s = 1.5, 0.75
    kc[0, 0, 1, 0] = c
    vc[0, 0, 0, :] = 2.0
    vc[0, 0, 1, :] = -4.0
    q = np.zeros((1, 1, d), np.float32)
    q[0, 0, 0] = 1.0
    out = decode(q, kc, vc, np.array([[0]]), np.array([2]), s, bs)
    e = math.exp(s * c)
    want = (2.0 - 4.0 * e) / (1.0 + e)
    np.testing.assert_allclose(out[0, 0], want, rtol=1e-14, atol=0)


def _random_case(seed, lens, hq, hkv, d, bs, pool, dtype=F32):
    rng = np.random.default_rng(seed)
    need = [-(-L // bs) for L in lens]
    maxb = max(max(need), 1)
    perm = rng.permutation(pool)
    tables = np.zeros((len(lens), maxb), np.int64)
    k = 0
    for i, n in enumerate(need):
        tables[i, :n] = perm[k:k + n]
        k += n
    kc = rng.standard_normal((pool, hkv, bs, d)).astype(np.float32)
    vc = rng.standard_normal((pool, hkv, bs, d)).astype(np.float32)
    q = rng.standard_normal((len(lens), hq, d)).astype(np.float32)
    return q, kc, vc, tables, np.array(lens)


def pin_library_sdpa(decode):
    """Contiguous physical layout (table = 0, 1, 2, ...) equals torch's float64
    scaled_dot_product_attention with the KV heads repeated per group."""
    bs, hq, hkv, d = 16, 8, 2, 32
    L = 100
    q, kc, vc, _, _ = _random_case(5, [L], hq, hkv, d, bs, 7)
    table = np.arange(7)[None, :]
    out = decode(q, kc, vc, table, np.array([L]), 0.2, bs)
    kk = torch.from_numpy(kc.astype(np.float64)).permute(1, 0, 2, 3).reshape(hkv, -1, d)[:, :L]
    vv = torch.from_numpy(vc.astype(np.float64)).permute(1, 0, 2, 3).reshape(hkv, -1, d)[:, :L]
    kk = kk.repeat_interleave(hq // hkv, dim=0)[None]
    vv = vv.repeat_interleave(hq // hkv, dim=0)[None]
    qq = torch.from_numpy(q.astype(np.float64))[:, :, None, :]
    ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, scale=0.2)[0, :, 0, :].numpy()
    np.testing.assert_allclose(out[0], ref, rtol=0, atol=1e-12)


def _brute_force(q, kc, vc, tables, lens, scale, bs):
    """Scalar-loop attention with math.exp; no numpy arithmetic."""
    s_n, hq, d = q.shape
    hkv = kc.shape[1]
    g = hq // hkv
    out = [[[0.0] * d for _ in range(hq)] for _ in range(s_n)]
    for s in range(s_n):
        L = int(lens[s])
        for h in range(hq):
            kv = h // g
            logits = []
            for t in range(L):
                pid = int(tables[s][t // bs])
                off = t % bs
                acc = 0.0
                for j in range(d):
                    acc += float(q[s, h, j]) * float(kc[pid, kv, off, j])
                logits.append(scale * acc)
            if L == 0:
                continue
            mx = max(logits)
            w = [math.exp(x - mx) for x in logits]
            tot = sum(w)
            for j in range(d):
                num = 0.0
                for t in range(L):
                    pid = int(tables[s][t // bs])
                    num += w[t] * float(vc[pid, kv, t % bs, j])
                out[s][h][j] = num / tot
    return np.array(out)


def pin_brute_force(decode):
    """Tiny-config shape (context lengths 1, 17, 100, 256 plus an empty one,
    block size 16, scattered blocks) against the scalar loop."""
    lens = [1, 17, 100, 0, 256]
    q, kc, vc, tables, lens_a = _random_case(6, lens, 4, 4, 16, 16, 40)
    out = decode(q, kc, vc, tables, lens_a, 0.25, 16)
    ref = _brute_force(q, kc, vc, tables, lens_a, 0.25, 16)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    assert np.all(out[3] == 0.0)


def pin_permutation_invariance(decode):
    """Relabelling the physical blocks (moving every block and rewriting the
    tables to match) changes nothing, bit for bit."""
    lens = [33, 64, 7]
    q, kc, vc, tables, lens_a = _random_case(7, lens, 4, 2, 16, 8, 30)
    base = decode(q, kc, vc, tables, lens_a, 0.3, 8)
    perm = np.random.default_rng(8).permutation(30)
    kc2 = np.empty_like(kc)
    vc2 = np.empty_like(vc)
    kc2[perm] = kc
    vc2[perm] = vc
    out = decode(q, kc2, vc2, perm[tables], lens_a, 0.3, 8)
    assert np.array_equal(base, out)
    # and a contiguous layout of the same rows gives the same value
    contig_k = np.zeros_like(kc)
    contig_v = np.zeros_like(vc)
    tab_c = np.zeros_like(tables)
    nxt = 0
    for i, L in enumerate(lens):
        for b in range(-(-L // 8)):
            contig_k[nxt] = kc[tables[i, b]]
            contig_v[nxt] = vc[tables[i, b]]
            tab_c[i, b] = nxt
            nxt += 1
    assert np.array_equal(base, decode(q, contig_k, contig_v, tab_c, lens_a, 0.3, 8))


def pin_prefix_sharing(decode):
    """Two sequences whose tables point at the same prefix blocks (reference
    count 2) read the same rows as a sequence whose prefix was copied into
    private blocks; with equal queries all three outputs are equal."""
    rng = np.random.default_rng(9)
    nb, hkv, bs, d = 12, 2, 4, 8
    kc = rng.standard_normal((nb, hkv, bs, d)).astype(np.float32)
    vc = rng.standard_normal((nb, hkv, bs, d)).astype(np.float32)
    kc2, vc2 = kc.copy(), vc.copy()  # logical copies of blocks 0, 1 into 5, 6
    kc2[5], kc2[6], vc2[5], vc2[6] = kc[0], kc[1], vc[0], vc[1]
    tables = np.array([[0, 1, 2], [0, 1, 2], [5, 6, 2]])
    qrow = rng.standard_normal((1, 4, d)).astype(np.float32)
    q = np.repeat(qrow, 3, axis=0)
    out = decode(q, kc2, vc2, tables, np.array([10, 10, 10]), 0.4, bs)
    assert np.array_equal(out[0], out[1]) and np.array_equal(out[0], out[2])


def pin_nan_poison(decode):
    """Slots past the context, unused blocks and padding table entries that
    point at a NaN block leave the output finite and unchanged."""
    lens = [5, 16, 23]
    q, kc, vc, tables, lens_a = _random_case(10, lens, 2, 2, 8, 8, 12)
    clean = decode(q, kc, vc, tables, lens_a, 0.5, 8)
    used = set()
    for i, L in enumerate(lens):
        used.update(int(x) for x in tables[i, :-(-L // 8)])
    trap = max(set(range(12)) - used)
    kp, vp = kc.copy(), vc.copy()
    tp = tables.copy()
    for i, L in enumerate(lens):
        nblk = -(-L // 8)
        tp[i, nblk:] = trap
        last = tables[i, nblk - 1]
        kp[last, :, L - (nblk - 1) * 8:, :] = np.nan
        vp[last, :, L - (nblk - 1) * 8:, :] = np.nan
    assert trap not in used
    for b in range(12):
        if b not in used:
            kp[b] = np.nan
            vp[b] = np.nan
    out = decode(q, kp, vp, tp, lens_a, 0.5, 8)
    assert np.all(np.isfinite(out)) and np.array_equal(out, clean)


PINS = [pin_slot_id_probe, pin_single_token, pin_zero_keys_give_mean, pin_gqa_head_mapping,
        pin_two_token_scale, pin_library_sdpa, pin_brute_force, pin_permutation_invariance,
        pin_prefix_sharing, pin_nan_poison]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_attention_pins(pin):
    pin(_decode)


def test_oracle_bf16_storage_matches_f32_values():
    """BF16 storage is decoded exactly: a bf16 cache and the float32 cache of
    the same values give the same float64 output."""
    q, kc, vc, tables, lens = _random_case(11, [9, 30], 4, 2, 16, 8, 10)
    to_bf = lambda a: torch.from_numpy(a).to(torch.bfloat16)
    qb, kb, vb = to_bf(q), to_bf(kc), to_bf(vc)
    out_b = oracle.paged_decode(qb.view(torch.uint16).numpy(), kb.view(torch.uint16).numpy(),
                                vstore(vb.view(torch.uint16).numpy()), tables, lens, 0.25, 8, BF16)
    out_f = oracle.paged_decode(qb.float().numpy(), kb.float().numpy(), vstore(vb.float().numpy()),
                                tables, lens, 0.25, 8, F32)
    assert np.array_equal(out_b, out_f)
    out_h = oracle.paged_decode(q.astype(np.float16), kc.astype(np.float16), vstore(vc.astype(np.float16)),
                                tables, lens, 0.25, 8, F16)
    ref_h = oracle.paged_decode(q.astype(np.float16).astype(np.float32),
                                kc.astype(np.float16).astype(np.float32),
                                vstore(vc.astype(np.float16).astype(np.float32)), tables, lens, 0.25, 8, F32)
    assert np.array_equal(out_h, ref_h)


# ---------------------------------------------------------------------------
# Planted mistakes: each mutant of the oracle must fail at least one pin
# ---------------------------------------------------------------------------

def _mutant(kind):
    def decode(q, kc, vc, tables, lens, scale, bs, dtype=F32):
        s_n, hq, d = q.shape
        hkv = kc.shape[1]
        g = hq // hkv
        out = np.zeros(q.shape)
        for s in range(s_n):
            L = int(lens[s])
            if kind == "ctx_off_by_one":
                L = min(L + 1, tables.shape[1] * bs)
            if L == 0:
                continue
            t = np.arange(L)
            if kind == "offset_wrong_axis":
                pid, off = tables[s][t % len(tables[s])], t // len(tables[s])
                off = np.minimum(off, bs - 1)
            else:
                pid, off = tables[s][t // bs], t % bs
            K = kc[pid, :, off, :].astype(np.float64)
            V = vc[pid, :, off, :].astype(np.float64)
            for h in range(hq):
                kv = h % hkv if kind == "head_modulo" else h // g
                sc = 1.0 if kind == "drop_scale" else scale
                x = sc * (K[:, kv, :] @ q[s, h].astype(np.float64))
                if kind == "sign":
                    x = -x
                p = np.exp(x - x.max())
                if kind == "transposed_v":
                    Vt = V[:, kv, :].reshape(-1)[: L * d].reshape(d, L).T if L == d else V[:, kv, ::-1]
                    out[s, h] = (p @ Vt) / p.sum()
                elif kind == "no_normalise":
                    out[s, h] = p @ V[:, kv, :]
                else:
                    out[s, h] = (p @ V[:, kv, :]) / p.sum()
        return out
    return decode


MUTANTS = ["ctx_off_by_one", "offset_wrong_axis", "head_modulo", "drop_scale", "sign",
           "transposed_v", "no_normalise"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_pins_catch_planted_mistake(kind):
    bad = _mutant(kind)
    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(bad)
        except (AssertionError, IndexError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches mutant {kind}"


def test_unmutated_copy_passes_all_pins():
    good = _mutant("none")
    for pin in PINS:
        pin(good)


# ---------------------------------------------------------------------------
# Split over partitions + log-sum-exp merge
# ---------------------------------------------------------------------------

def test_lse_merge_equals_unsplit_softmax():
    lens = [1, 16, 17, 100, 513, 1030, 0]
    q, kc, vc, tables, lens_a = _random_case(12, lens, 4, 2, 16, 16, 120)
    ref = oracle.paged_decode(q, kc, vstore(vc), tables, lens_a, 0.3, 16, F32)
    for part in (16, 48, 512, 4096):
        got = oracle.paged_decode_partitioned(q, kc, vstore(vc), tables, lens_a, 0.3, 16, F32, part)
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_lse_merge_single_and_empty_partitions():
    rng = np.random.default_rng(13)
    o = rng.standard_normal(8)
    one = oracle.lse_merge([(0.7, 3.0, o)])
    np.testing.assert_allclose(one, o, rtol=1e-15, atol=0)  # (3 o) / 3, one rounding
    empty = (-math.inf, 0.0, np.zeros(8))
    two = oracle.lse_merge([empty, (0.7, 3.0, o), empty])
    assert np.array_equal(two, one)
    assert np.array_equal(oracle.lse_merge([empty, empty]), np.zeros(8))
    m, l_sum, o_e = oracle.partition_stats(o, np.zeros((0, 8)), np.zeros((0, 8)), 1.0)
    assert m == -math.inf and l_sum == 0.0 and np.all(o_e == 0)


def test_partition_stats_closed_form():
    # keys [0, 1] along e0, query e0, scale 1: logits [0, 1]
    k = np.array([[0.0, 0.0], [1.0, 0.0]])
    v = np.array([[1.0, 0.0], [0.0, 1.0]])
    m, l_sum, o = oracle.partition_stats(np.array([1.0, 0.0]), k, v, 1.0)
    assert m == 1.0
    assert math.isclose(l_sum, 1.0 + math.exp(-1.0), rel_tol=1e-15)
    np.testing.assert_allclose(o, [math.exp(-1) / (1 + math.exp(-1)), 1 / (1 + math.exp(-1))], rtol=1e-15)


# ---------------------------------------------------------------------------
# Cache write and block copy
# ---------------------------------------------------------------------------

def test_write_probe_worked_example():
    """Position 9 of a sequence with table [5, 1, 7] and B = 4 goes to slot
    7 * 4 + 1 = 29, i.e. cache[7, :, 1, :]; nothing else changes."""
    c = _golden("block_layout.json")["translate_case"]
    nb, hkv, bs, d = 8, 2, c["block_size"], 8
    rng = np.random.default_rng(14)
    kc = rng.integers(0, 2 ** 16, (nb, hkv, bs, d), dtype=np.uint16)
    vl = rng.integers(0, 2 ** 16, (nb, hkv, bs, d), dtype=np.uint16)
    vc = vstore(vl)
    k = rng.integers(0, 2 ** 16, (1, hkv, d), dtype=np.uint16)
    v = rng.integers(0, 2 ** 16, (1, hkv, d), dtype=np.uint16)
    logical, off = divmod(c["position"], bs)
    slot = c["block_table"][logical] * bs + off
    assert slot == 29
    k2, v2 = oracle.write_cache(k, v, kc, vc, [slot], bs)
    want_v = vl.copy()
    want_v[7, :, 1, :] = v[0]
    assert np.array_equal(k2[7, :, 1, :], k[0]) and np.array_equal(v2, vstore(want_v))
    mask = np.ones(kc.shape, bool)
    mask[7, :, 1, :] = False
    assert np.array_equal(k2[mask], kc[mask])


def test_write_skips_negative_slot_and_keeps_raw_bits():
    nb, hkv, bs, d = 4, 1, 4, 4
    kc = np.zeros((nb, hkv, bs, d), np.uint16)
    vc = np.zeros(oracle.v_cache_shape(nb, hkv, bs, d), np.uint16)
    # NaN payloads, signed zero, infinity: moved as bits
    k = np.array([[[0x7FC1, 0xFFFF, 0x8000, 0x7F80]], [[1, 2, 3, 4]]], np.uint16)
    v = np.array([[[0x7F81, 0x0001, 0xFF80, 0x3F80]], [[5, 6, 7, 8]]], np.uint16)
    k2, v2 = oracle.write_cache(k, v, kc, vc, [13, -1], bs)
    assert np.array_equal(k2[3, 0, 1], k[0, 0]) and np.array_equal(v2[3, 0, 0, :, 1], v[0, 0])
    assert int(k2.astype(np.int64).sum()) == int(k[0].astype(np.int64).sum())


def test_write_preconditions():
    kc = np.zeros((2, 1, 4, 2), np.float32)
    vc = np.zeros(oracle.v_cache_shape(2, 1, 4, 2), np.float32)
    k = np.ones((2, 1, 2), np.float32)
    with pytest.raises(ValueError):
        oracle.write_cache(k, k, kc, vc, [3, 3], 4)
    with pytest.raises(IndexError):
        oracle.write_cache(k, k, kc, vc, [8, 1], 4)
    with pytest.raises(IndexError):
        oracle.write_cache(k, k, kc, vc, [-2, 1], 4)
    with pytest.raises(ValueError):
        oracle.write_cache(k, k, kc, kc, [0, 1], 4)  # V in the untransposed shape


def test_copy_blocks_whole_block_and_source_untouched():
    rng = np.random.default_rng(15)
    kc = rng.integers(0, 2 ** 16, (6, 2, 4, 3), dtype=np.uint16)
    vc = rng.integers(0, 2 ** 16, oracle.v_cache_shape(6, 2, 4, 3), dtype=np.uint16)
    k2, v2 = oracle.copy_blocks(kc, vc, [[1, 4], [2, 5]])
    assert np.array_equal(k2[4], kc[1]) and np.array_equal(k2[5], kc[2])
    assert np.array_equal(v2[4], vc[1]) and np.array_equal(v2[5], vc[2])
    for b in (0, 1, 2, 3):
        assert np.array_equal(k2[b], kc[b]) and np.array_equal(v2[b], vc[b])
    k3, v3 = oracle.copy_blocks(kc, vc, np.zeros((0, 2), np.int64))
    assert np.array_equal(k3, kc) and np.array_equal(v3, vc)


def test_copy_blocks_preconditions():
    kc = np.zeros((4, 1, 2, 2), np.float32)
    with pytest.raises(ValueError):
        oracle.copy_blocks(kc, kc, [[0, 1], [2, 1]])
    with pytest.raises(ValueError):
        oracle.copy_blocks(kc, np.zeros((5, 1, 1, 2, 2), np.float32), [[0, 1]])
    with pytest.raises(ValueError):
        oracle.copy_blocks(kc, kc, [[0, 1], [1, 2]])
    with pytest.raises(IndexError):
        oracle.copy_blocks(kc, kc, [[0, 4]])


def test_cow_isolates_writer_from_sharers():
    """Copy-on-write: after copying the shared block and writing the new token
    into the copy, the sharers' rows and outputs are unchanged bit for bit."""
    rng = np.random.default_rng(16)
    nb, hkv, bs, d = 8, 1, 4, 8
    kc = rng.standard_normal((nb, hkv, bs, d)).astype(np.float32)
    vc = rng.standard_normal((nb, hkv, bs, d)).astype(np.float32)
    q = rng.standard_normal((2, 2, d)).astype(np.float32)
    tables = np.array([[0, 1], [0, 1]])  # both share blocks 0 and 1 (block 1 half full)
    vc = vstore(vc)
    before = oracle.paged_decode(q, kc, vc, tables, np.array([6, 6]), 0.3, bs, F32)
    k2, v2 = oracle.copy_blocks(kc, vc, [[1, 5]])
    new_k = rng.standard_normal((1, hkv, d)).astype(np.float32)
    k3, v3 = oracle.write_cache(new_k, new_k, k2, v2, [5 * bs + 2], bs)
    tables2 = np.array([[0, 1], [0, 5]])
    after = oracle.paged_decode(q, k3, v3, tables2, np.array([6, 7]), 0.3, bs, F32)
    assert np.array_equal(after[0], before[0])
    assert np.array_equal(k3[1], kc[1]) and np.array_equal(v3[1], vc[1])
    assert not np.array_equal(after[1], before[1])


def test_v_layout_reading():
    """The transposed tile layout: the V row of (pid, off) is
    v_cache[pid, :, off // T, :, off % T] with T = min(B, 16). Writing every
    slot through write_cache and reading every row back through gather_rows
    are inverse maps of the test-side conversion, for block sizes below, at
    and above the tile."""
    rng = np.random.default_rng(17)
    for bs in (4, 8, 16, 32, 64):
        nb, hkv, d = 3, 2, 8
        vl = rng.integers(0, 2 ** 16, (nb, hkv, bs, d), dtype=np.uint16)
        store = vstore(vl)
        assert store.shape == oracle.v_cache_shape(nb, hkv, bs, d)
        # element (pid, kv, off, dd) sits at flat index
        # (((pid * hkv + kv) * (B / T) + off // T) * D + dd) * T + off % T
        t = min(bs, 16)
        flat = store.reshape(-1)
        for (pid, kv, off, dd) in [(0, 0, 0, 0), (2, 1, bs - 1, d - 1), (1, 0, bs // 2, 3)]:
            idx = (((pid * hkv + kv) * (bs // t) + off // t) * d + dd) * t + off % t
            assert flat[idx] == vl[pid, kv, off, dd]
        slots = np.arange(nb * bs)
        k = np.zeros((nb * bs, hkv, d), np.uint16)
        v = vl.transpose(0, 2, 1, 3).reshape(nb * bs, hkv, d)
        _, v_written = oracle.write_cache(k, v, np.zeros((nb, hkv, bs, d), np.uint16),
                                          np.zeros_like(store), slots, bs)
        assert np.array_equal(v_written, store)
        rows = oracle.gather_rows(store, [2, 0, 1], 3 * bs, bs, BF16, "v")
        want = oracle.to_float64(np.concatenate([vl[2], vl[0], vl[1]], axis=1).transpose(1, 0, 2), BF16)
        assert np.array_equal(rows, want, equal_nan=True)
