"""GPU properties and edge cases of the decode path, each against the CPU
oracle or against a bitwise invariant that needs no oracle:
dtype x head_dim x group matrix, partition sizes (split-K and merge),
permutation invariance and shared-vs-copied blocks (bitwise), run-to-run
determinism, empty sequences, context-length and table-entry clamping,
the largest supported batch."""

import numpy as np
import pytest
import torch

import oracle
from harness import ORACLE_DTYPE, compare_attention, host_bits, log

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_165_amd as pa
    pa.library()


def _pa():
    import paged_kv_cache_165_amd as pa
    return pa


def make_case(lens, hq, hkv, d, bs, dtype, seed, pool=None, trap_nan=True):
    """Scattered blocks, NaN in every slot that is not part of a context."""
    rng = np.random.default_rng(seed)
    need = [-(-int(L) // bs) for L in lens]
    total = sum(need)
    nb = pool or max(total + 2, int(total * 1.25) + 2)
    perm = rng.permutation(nb)
    trap = int(perm[-1])
    maxb = max(max(need), 1)
    tables = np.full((len(lens), maxb), trap, np.int32)
    valid = np.zeros((nb, bs), bool)
    k = 0
    for i, (L, n) in enumerate(zip(lens, need)):
        tables[i, :n] = perm[k:k + n]
        for t in range(int(L)):
            valid[tables[i, t // bs], t % bs] = True
        k += n
    g = torch.Generator(device=DEV).manual_seed(seed)
    rn = lambda *s: torch.randn(*s, generator=g, device=DEV).to(dtype)
    t = min(bs, 16)
    q = rn(len(lens), hq, d)
    kc = rn(nb, hkv, bs, d)
    vc = rn(nb, hkv, bs // t, d, t)   # transposed V tiles
    if trap_nan:
        m = torch.from_numpy(valid).to(DEV)
        nan = torch.full((), float("nan"), dtype=dtype, device=DEV)
        kc = torch.where(m.view(nb, 1, bs, 1), kc, nan)
        vc = torch.where(m.view(nb, 1, bs // t, 1, t), vc, nan)
    return dict(q=q, kc=kc, vc=vc, tables=tables, lens=np.array(lens, np.int32), bs=bs)


def run_gpu(c, scale, part=0, max_ctx=None, tables=None, lens=None, kc=None, vc=None):
    pa = _pa()
    tables = c["tables"] if tables is None else tables
    lens = c["lens"] if lens is None else lens
    t_d = torch.from_numpy(np.ascontiguousarray(tables)).to(DEV)
    l_d = torch.from_numpy(np.ascontiguousarray(lens)).to(DEV)
    mc = int(lens.max()) if max_ctx is None else max_ctx
    out = torch.empty_like(c["q"])
    pa.decode(out, c["q"], c["kc"] if kc is None else kc, c["vc"] if vc is None else vc, t_d, l_d,
              scale, max_context_len=mc, partition_size=part)
    torch.cuda.synchronize()
    return out


def run_oracle(c, scale, lens=None):
    dt = ORACLE_DTYPE[c["q"].dtype]
    lens = c["lens"] if lens is None else lens
    return oracle.paged_decode(host_bits(c["q"]), host_bits(c["kc"]), host_bits(c["vc"]), c["tables"],
                               lens, scale, c["bs"], dt)


MATRIX = [(dt, d, g) for dt in (torch.float32, torch.bfloat16, torch.float16)
          for d in (64, 128, 256) for g in (1, 2, 4, 8)]


MATRIX += [(torch.bfloat16, d, 16) for d in (64, 128, 256)] + [(torch.float16, 128, 16)]


@pytest.mark.parametrize("dt,d,g", MATRIX, ids=[f"{str(dt)[6:]}-D{d}-g{g}" for dt, d, g in MATRIX])
def test_dtype_headdim_group_matrix(dt, d, g):
    hkv = 2
    lens = [1, 15, 16, 17, 300, 700, 1500]
    c = make_case(lens, hkv * g, hkv, d, 16, dt, seed=d * 10 + g)
    scale = 1.0 / np.sqrt(d)
    out = run_gpu(c, scale)
    stats = compare_attention(out, run_oracle(c, scale), f"{dt} D{d} g{g}")
    log(f"[matrix] {dt} D{d} g{g}: {stats}")


@pytest.mark.parametrize("part", [16, 32, 64, 256, 512, 1024, 4096])
def test_partition_sizes(part):
    lens = [1, 16, 33, 511, 512, 513, 2000, 4100]
    c = make_case(lens, 16, 4, 128, 16, torch.bfloat16, seed=part)
    out = run_gpu(c, 0.09, part=part)
    compare_attention(out, run_oracle(c, 0.09), f"part {part}")


@pytest.mark.parametrize("dt,g", [(torch.bfloat16, 4), (torch.bfloat16, 1), (torch.float32, 2)])
def test_full_table_slice_partitions(dt, g):
    """Partitions of 512 blocks, the most one item stages (two table entries
    per thread), with sequences just under, at and over one and two of them,
    and the library's default split on the same batch."""
    lens = [8191, 8192, 8193, 16385, 40]
    c = make_case(lens, 2 * g, 2, 128, 16, dt, seed=513 + g)
    ref = run_oracle(c, 0.07)
    compare_attention(run_gpu(c, 0.07, part=8192), ref, f"{dt} g{g} part 8192")
    compare_attention(run_gpu(c, 0.07, part=0), ref, f"{dt} g{g} default partition")


@pytest.mark.parametrize("bs", [4, 8, 16, 32])
@pytest.mark.parametrize("dt,g", [(torch.bfloat16, 4), (torch.float16, 8)])
def test_stream_and_workgroup_mfma_kernels(dt, g, bs):
    """16-bit grouped heads run the stream split when a partition spans at
    most 128 blocks and one item per workgroup above that: both, at every
    small block size, and the library's default split."""
    lens = [1, 5, 16, 31, 700, 2049, 5000]
    c = make_case(lens, 2 * g, 2, 128, bs, dt, seed=40 + bs + g)
    ref = run_oracle(c, 0.08)
    for part, kind in ((128 * bs, "stream"), (256 * bs, "workgroup"), (0, "default")):
        compare_attention(run_gpu(c, 0.08, part=part), ref, f"{dt} g{g} bs{bs} part {part} ({kind})")


def test_wave_items_past_the_stream_cost_bound():
    """The stream split keeps its cost positions in 32 bits, so a batch that
    could pass 2^31 runs one item per wave instead. The bound is taken on
    max_context_len, so 1024 short sequences of 8 KV heads declared up to
    2^20 tokens reach it (blocks of 128 keep the table at 8192 entries per
    sequence; table entries past each context are never read)."""
    pa = _pa()
    n, hkv, g, bs, mc, part = 1024, 8, 4, 128, 2 ** 20, 16384
    assert n * hkv * (4 * (mc // 16) + 3) >= 2 ** 31 - 1
    plan = pa.decode_plan(n, hkv * g, hkv, 128, mc, bs, part, torch.bfloat16)
    assert plan["kernel"] == "mfma_wave", plan
    lens = np.random.default_rng(77).integers(0, bs + 1, size=n)
    lens[:3] = [0, 1, bs]
    c = make_case(lens, hkv * g, hkv, 128, bs, torch.bfloat16, seed=77)
    wide = np.zeros((n, mc // bs), np.int32)
    wide[:, :c["tables"].shape[1]] = c["tables"]
    out = run_gpu(c, 0.09, part=part, max_ctx=mc, tables=wide)
    compare_attention(out, run_oracle(c, 0.09), "wave items past the stream cost bound")


@pytest.mark.parametrize("bs", [4, 8, 16, 32, 64, 128, 256])
@pytest.mark.parametrize("g", [1, 4])
def test_block_sizes(bs, g):
    lens = [3, 64, 129, 1000, 2049]
    c = make_case(lens, 2 * g, 2, 128, bs, torch.bfloat16, seed=bs + g)
    part = max(512, bs)
    out = run_gpu(c, 0.09, part=part)
    compare_attention(out, run_oracle(c, 0.09), f"bs {bs} g {g}")


@pytest.mark.parametrize("bs", [8, 16, 32])
@pytest.mark.parametrize("dt,d", [(torch.float32, 128), (torch.float32, 256), (torch.bfloat16, 256),
                                  (torch.bfloat16, 64), (torch.float16, 64)])
def test_block_sizes_wide_rows(bs, dt, d):
    """Row geometries other than 256-byte rows with one query head per KV
    head: the VALU kernel for float32, the stream split for 16-bit elements.
    float32 head_dim 256 takes blocks of at least 16 tokens: a smaller block
    is rejected with PA_ERR_UNSUPPORTED before anything is launched."""
    c = make_case([5, 100, 700], 4, 4, d, bs, dt, seed=bs + d)
    if dt == torch.float32 and d == 256 and bs < 16:
        pa = _pa()
        with pytest.raises(pa.PaError) as e:
            run_gpu(c, 0.1)
        assert e.value.status == pa._lib.PA_ERR_UNSUPPORTED
        return
    out = run_gpu(c, 0.1)
    compare_attention(out, run_oracle(c, 0.1), f"{dt} D{d} bs {bs}")


@pytest.mark.parametrize("bs,hq,hkv", [(16, 32, 8), (8, 32, 8), (4, 8, 8)])
def test_permutation_invariance_bitwise(bs, hq, hkv):
    """Moving every block to another physical id (tables rewritten to match)
    gives bit-identical outputs: the reduction order depends only on logical
    positions. Blocks of 16 (wave-uniform bases), of 8 and 4 (each lane's own
    block ids; one query head per KV head at 4)."""
    lens = [5, 400, 1030, 3000]
    c = make_case(lens, hq, hkv, 128, bs, torch.bfloat16, seed=7 + bs)
    base = run_gpu(c, 0.09)
    nb = c["kc"].shape[0]
    perm = np.random.default_rng(8).permutation(nb)
    inv = torch.from_numpy(np.argsort(perm)).to(DEV)
    kc2 = c["kc"][inv].contiguous()   # block b moves to perm[b]
    vc2 = c["vc"][inv].contiguous()
    out2 = run_gpu(c, 0.09, tables=perm[c["tables"]].astype(np.int32), kc=kc2, vc=vc2)
    assert torch.equal(base.view(torch.int16), out2.view(torch.int16))


@pytest.mark.parametrize("bs,g", [(16, 4), (32, 1), (8, 4)])
def test_shared_blocks_hint_changes_nothing_but_the_loads(bs, g):
    """decode with the shared-blocks hint (pa_decode_ex) equals the plain
    call bit for bit, on sequences whose tables share a prefix (four samples
    of each of three prompts) and on blocks of 8, where the hint is ignored."""
    pa = _pa()
    hkv = 4
    lens = [900, 1300, 700, 2000, 1000, 800]
    c = make_case(lens, hkv * g, hkv, 128, bs, torch.bfloat16, seed=31 + bs + g, trap_nan=False)
    tables = c["tables"].copy()
    share = 512 // bs
    for i in range(len(lens)):                  # sequence i shares its first 512 tokens with sequence i % 2
        tables[i, :share] = c["tables"][i % 2, :share]
    q = c["q"]
    t_d = torch.from_numpy(tables).to(DEV)
    l_d = torch.from_numpy(c["lens"]).to(DEV)
    mc = int(c["lens"].max())
    plain = torch.empty_like(q)
    hinted = torch.empty_like(q)
    pa.decode(plain, q, c["kc"], c["vc"], t_d, l_d, 0.08, max_context_len=mc)
    pa.decode(hinted, q, c["kc"], c["vc"], t_d, l_d, 0.08, max_context_len=mc, shared_blocks=True)
    torch.cuda.synchronize()
    assert torch.equal(plain.view(torch.int16), hinted.view(torch.int16))
    c2 = dict(c, tables=tables)
    compare_attention(hinted, run_oracle(c2, 0.08), f"shared-blocks hint bs {bs} g {g}")


def test_shared_blocks_equal_copied_blocks_bitwise():
    """Sequences whose tables share prefix blocks (reference count 3) and a
    sequence reading copies of those blocks made by pa_copy_blocks give the
    same output bit for bit when their queries are equal."""
    pa = _pa()
    bs, hkv, d = 16, 8, 128
    c = make_case([700], 32, hkv, d, bs, torch.bfloat16, seed=9, pool=200, trap_nan=False)
    nblk = -(-700 // bs)
    row = c["tables"][0, :nblk]
    free = np.setdiff1d(np.arange(200), row)[:nblk]
    pairs = torch.from_numpy(np.stack([row, free], 1).astype(np.int32)).to(DEV)
    pa.copy_blocks(c["kc"], c["vc"], pairs)
    tables = np.stack([row, row, row, free]).astype(np.int32)
    q = c["q"].expand(4, -1, -1).contiguous()
    c4 = dict(c, q=q)
    out = run_gpu(c4, 0.09, tables=tables, lens=np.array([700] * 4, np.int32))
    for i in range(1, 4):
        assert torch.equal(out[0].view(torch.int16), out[i].view(torch.int16))


def test_deterministic_repeat():
    c = make_case([17, 900, 5000], 64, 8, 128, 32, torch.bfloat16, seed=10)
    a = run_gpu(c, 0.09)
    b = run_gpu(c, 0.09)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_empty_sequences_give_zero_rows():
    c = make_case([0, 40, 0, 1300, 0], 8, 2, 128, 16, torch.bfloat16, seed=11)
    out = run_gpu(c, 0.09)
    assert torch.all(out[0] == 0) and torch.all(out[2] == 0) and torch.all(out[4] == 0)
    compare_attention(out, run_oracle(c, 0.09), "empty")
    c2 = make_case([0, 0], 8, 2, 128, 16, torch.bfloat16, seed=12)
    out2 = run_gpu(c2, 0.09, max_ctx=0)
    assert torch.all(out2 == 0)


def test_context_longer_than_bound_is_clamped():
    """A context length above max_context_len is read as max_context_len
    tokens (documented clamp), never past the bound."""
    c = make_case([100, 600, 900], 8, 2, 128, 16, torch.bfloat16, seed=13)
    out = run_gpu(c, 0.09, max_ctx=600)
    ref = run_oracle(c, 0.09, lens=np.minimum(c["lens"], 600))
    compare_attention(out, ref, "clamp")


def test_out_of_range_table_entries_do_not_fault():
    c = make_case([50, 300], 8, 2, 128, 16, torch.bfloat16, seed=14, trap_nan=False)
    t = c["tables"].copy()
    t[0, 1] = 10 ** 8
    t[1, 3] = -5
    out = run_gpu(c, 0.09, tables=t)
    assert torch.all(torch.isfinite(out.float()))


def test_largest_batch():
    lens = np.random.default_rng(15).integers(1, 64, size=8192)
    c = make_case(lens.tolist(), 8, 2, 64, 16, torch.bfloat16, seed=15)
    out = run_gpu(c, 0.125)
    compare_attention(out, run_oracle(c, 0.125), "8192 seqs")


def test_shape_beyond_the_lds_is_refused_before_launch():
    """A valid shape whose launch plan does not fit the compute unit's LDS
    (8192 sequences, 16 query heads per KV head, head_dim 256: the stream
    split's schedule and query blocks) is refused with PA_ERR_UNSUPPORTED on
    the host, naming the LDS, and nothing is launched: the output keeps its
    contents. The same shape with fewer sequences runs."""
    import paged_kv_cache_165_amd as pa
    from paged_kv_cache_165_amd import _lib
    s, hkv, g, d, bs = 8192, 2, 16, 256, 16
    with pytest.raises(pa.PaError):
        pa.decode_plan(s, hkv * g, hkv, d, 1, bs, 0, torch.bfloat16)
    q = torch.zeros(s, hkv * g, d, dtype=torch.bfloat16, device=DEV)
    kc, vc = pa.alloc_cache(s, hkv, bs, d, dtype=torch.bfloat16, device=DEV)
    kc.zero_()
    vc.zero_()
    tables = torch.arange(s, dtype=torch.int32, device=DEV).view(s, 1)
    lens = torch.ones(s, dtype=torch.int32, device=DEV)
    out = torch.full_like(q, 7.0)
    with pytest.raises(pa.PaError) as err:
        pa.decode(out, q, kc, vc, tables, lens, 0.0625, max_context_len=1)
    assert err.value.status == _lib.PA_ERR_UNSUPPORTED and "LDS" in str(err.value)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
    n = 1024
    pa.decode(out[:n], q[:n], kc, vc, tables[:n], lens[:n], 0.0625, max_context_len=1)
    torch.cuda.synchronize()
    assert bool((out[:n] == 0).all()) and bool((out[n:] == 7.0).all())


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
def test_one_pair_split_over_every_wave(dt):
    """One (sequence, KV head) pair of 65,536 tokens: the stream split gives
    every wave of the grid a stretch of it, so the merge combines one tail
    record with about a thousand head records (its chunked loads, 32 at a
    time)."""
    pa = _pa()
    plan = pa.decode_plan(1, 4, 1, 128, 65536, 16, 0, dt)
    assert plan["kernel"] == "mfma_stream"
    c = make_case([65536], 4, 1, 128, 16, dt, seed=16)
    compare_attention(run_gpu(c, 0.088), run_oracle(c, 0.088), "one pair, every wave")


def test_stream_mixes_tiny_and_long_pairs():
    """Hundreds of one- to three-token sequences around a few long ones:
    waves that hold many whole pairs write them directly, the long pairs are
    split between waves, and empty sequences sit between them."""
    rng = np.random.default_rng(17)
    lens = rng.integers(0, 4, size=900)
    lens[[5, 450, 899]] = [30000, 17, 45000]
    c = make_case(lens.tolist(), 32, 8, 128, 16, torch.bfloat16, seed=17)
    pa = _pa()
    assert pa.decode_plan(900, 32, 8, 128, 45000, 16, 0, torch.bfloat16)["kernel"] == "mfma_stream"
    compare_attention(run_gpu(c, 0.088), run_oracle(c, 0.088), "tiny and long")
