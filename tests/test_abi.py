"""The C-ABI library loads, exports every function include/pa.h declares, and
rejects bad arguments on the host before anything is launched. No GPU: only
validation paths are called, none of which touches the device."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("pa.h", "pa_blocks.h", "pa_probe.h")]


def _lib():
    from paged_kv_cache_165_amd import _lib as L
    if not os.path.exists(L.LIB_PATH):
        pytest.skip("libpa.so not built (run __graft_entry__.build())")
    return L.load(), L


def _declared():
    names = set()
    for h in HEADERS:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names.update(re.findall(r"\b(pa_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


def test_header_declares_expected_entry_points():
    names = _declared()
    for n in ("pa_decode", "pa_prefill", "pa_write_cache", "pa_copy_blocks", "pa_decode_workspace_size"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib, L = _lib()
    names = _declared()
    assert set(names) == set(L.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.pa_abi_version() == 10


def test_status_strings_and_workspace_size():
    lib, L = _lib()
    assert lib.pa_status_string(0) == b"ok"
    assert lib.pa_status_string(3) == b"workspace missing or too small"
    dp = lib.pa_default_partition_size
    F32, BF16, F16 = 0, 1, 2
    # workgroup items (float32): 256 blocks, halved while the batch has < 512
    # items, not below 512 tokens
    assert dp(64, 32, 32, 4096, 16, F32) == 4096      # 2048 pairs, one partition each
    assert dp(256, 8, 8, 8192, 16, F32) == 4096
    assert dp(8, 8, 8, 131072, 32, F32) == 8192       # 64 pairs x 16 partitions = 1024 items
    assert dp(1, 8, 8, 131072, 16, F32) == 2048       # 8 pairs: halve until 8 x 64 = 512 items
    assert dp(4, 4, 4, 256, 16, F32) == 512           # tiny batch: floor of 512 tokens
    assert dp(64, 8, 8, 1000, 4, F32) == 1024         # 256 blocks of 4; 512 pairs suffice
    assert dp(32, 8, 8, 1000, 4, F32) == 512          # 256 pairs: halved once
    assert dp(2, 1, 1, 4096, 256, F32) == 512
    # 16-bit elements (the stream split, or wave items): min(2048, 128
    # blocks), halved while < 2048 items
    assert dp(256, 32, 8, 8192, 16, BF16) == 2048     # 2048 pairs x 4 partitions
    assert dp(64, 32, 32, 4096, 16, BF16) == 2048     # one query head per KV head: 2048 pairs x 2
    assert dp(8, 8, 8, 131072, 32, BF16) == 2048      # 64 pairs x 64 partitions
    assert dp(64, 8, 8, 1000, 4, BF16) == 512         # 128 blocks of 4, 512 pairs: the floor
    assert dp(2, 1, 1, 4096, 256, BF16) == 512        # 2 pairs: halve to the floor
    assert dp(8, 64, 8, 131072, 32, BF16) == 2048     # 64 pairs x 64 partitions
    assert dp(1, 64, 8, 131072, 32, F16) == 512       # 8 pairs: halve to the floor
    assert dp(256, 32, 8, 1000, 8, BF16) == 1024      # 128 blocks of 8
    assert dp(256, 32, 8, 1000, 4, BF16) == 512       # 128 blocks of 4
    assert dp(64, 32, 8, 2000, 16, BF16) == 512       # 512 pairs: halve until 512 x 4 items
    for bad in [(-1, 8, 8, 100, 16, 1), (1, 8, 0, 100, 16, 1), (1, 8, 8, 100, 0, 1), (1, 8, 3, 100, 16, 1),
                (1, 8, 8, 100, 16, 7)]:
        assert dp(*bad) == 0, bad
    # single partition: no workspace needed (item kernels)
    assert lib.pa_decode_workspace_size(4, 8, 8, 128, 512, 16, 0, F32) == 0
    assert lib.pa_decode_workspace_size(4, 8, 8, 128, 1024, 16, 1024, F32) == 0
    assert lib.pa_decode_workspace_size(4, 8, 8, 128, 512, 8, 0, F32) == 0
    # records of (m, l, o[D]) floats, each region 256-byte aligned
    recs = 4 * 8 * 3
    a = lambda x: (x + 255) // 256 * 256
    expect = a(recs * 4) * 2 + a(recs * 128 * 4)
    assert lib.pa_decode_workspace_size(4, 8, 2, 128, 1100, 16, 512, F32) == expect
    # the default resolves as pa_default_partition_size does: 4 x 2 pairs, 1100 tokens -> 512
    assert lib.pa_decode_workspace_size(4, 8, 2, 128, 1100, 16, 0, F32) == expect
    # 16-bit elements run the stream split: no
    # per-partition records; per wave of the grid's 1024, a tail and a head
    # record of every query head of a group and four ints naming the pair
    # of the tail record, whatever the batch and the partition
    xrecs = 2 * 1024 * 4
    stream = a(1024 * 16) + 2 * a(xrecs * 4) + a(xrecs * 128 * 4)
    assert lib.pa_decode_workspace_size(4, 8, 2, 128, 1100, 16, 512, BF16) == stream
    assert lib.pa_decode_workspace_size(4, 8, 2, 128, 1100, 16, 0, BF16) == stream
    assert lib.pa_decode_workspace_size(4, 8, 2, 128, 500, 16, 512, BF16) == stream
    # one query head per KV head runs it too, and so do blocks of 8
    x1 = 2 * 1024 * 1
    assert lib.pa_decode_workspace_size(4, 8, 8, 128, 512, 16, 0, BF16) == \
        a(1024 * 16) + 2 * a(x1 * 4) + a(x1 * 128 * 4)
    assert lib.pa_decode_workspace_size(4, 8, 2, 128, 1100, 8, 512, BF16) == stream
    # a batch whose stream cost positions could pass 2^31 (1024 x 8 pairs of
    # up to 2^20 tokens) keeps the one-item-per-wave kernel and its records
    big = 1024 * 32 * 64
    assert lib.pa_decode_workspace_size(1024, 32, 8, 128, 2 ** 20, 128, 16384, BF16) == \
        a(big * 4) * 2 + a(big * 128 * 4)
    assert lib.pa_decode_workspace_size(-1, 8, 8, 128, 1100, 16, 0, BF16) == 0
    assert lib.pa_decode_workspace_size(4, 8, 8, 128, 1100, 16, 0, 9) == 0


def _decode(lib, **over):
    args = dict(out=16, q=32, k=48, v=64, tables=80, lens=96, scale=0.1, bs=16, S=2, Hq=8, Hkv=2, D=128,
                NB=10, maxblk=4, maxctx=64, part=0, dtype=1, ws=0, ws_bytes=0, stream=None)
    args.update(over)
    return lib.pa_decode(args["out"], args["q"], args["k"], args["v"], args["tables"], args["lens"],
                         args["scale"], args["bs"], args["S"], args["Hq"], args["Hkv"], args["D"], args["NB"],
                         args["maxblk"], args["maxctx"], args["part"], args["dtype"], args["ws"],
                         args["ws_bytes"], args["stream"])


@pytest.mark.parametrize("over,status,msg", [
    (dict(Hq=7), 1, b"multiple of num_kv_heads"),
    (dict(Hq=64, Hkv=2), 2, b"no kernel"),          # group 32
    (dict(Hq=32, Hkv=2, dtype=0), 2, b"no kernel"), # float32 group 16
    (dict(D=96), 2, b"no kernel"),
    (dict(bs=12), 2, b"power of two"),
    (dict(bs=0), 1, b"zero size"),
    (dict(S=-1), 1, b"zero size"),
    (dict(maxblk=3), 1, b"max_blocks_per_seq"),      # 3 * 16 < 64
    (dict(part=24), 1, b"partition_size"),
    (dict(part=16 * 513), 1, b"partition_size"),    # 513 blocks: one more than an item stages
    (dict(dtype=7), 1, b"unknown dtype"),
    (dict(q=0), 1, b"null pointer"),
    (dict(out=8), 1, b"16-byte aligned"),
    (dict(maxctx=3000, maxblk=200), 3, b"workspace"),
    (dict(scale=float("inf")), 1, b"scale"),
    (dict(S=9000), 2, b"num_seqs"),
])
def test_decode_rejects_before_launch(over, status, msg):
    lib, _ = _lib()
    assert _decode(lib, **over) == status
    assert msg in lib.pa_last_error()


@pytest.mark.parametrize("name", ["pa_decode_ex", "pa_decode_partitions_ex"])
@pytest.mark.parametrize("flags", [2, 0x80000000, 3])
def test_decode_ex_rejects_unknown_flags_before_launch(name, flags):
    """Only PA_DECODE_SHARED_BLOCKS is defined: any other bit is refused
    after the shape checks and before a launch (the pointers here are never
    dereferenced), and so is a malformed shape whatever the flags."""
    lib, L = _lib()
    f = getattr(lib, name)
    a = (16, 32, 48, 64, 80, 96, 0.1, 16, 2, 8, 2, 128, 10, 4, 64, 0, 1, 128, 1 << 30)
    assert f(*a, flags, None) == L.PA_ERR_INVALID_ARG
    assert b"unknown decode flags" in lib.pa_last_error()
    bad = a[:9] + (7,) + a[10:]      # 7 query heads over 2 KV heads
    assert f(*bad, L.PA_DECODE_SHARED_BLOCKS, None) == L.PA_ERR_INVALID_ARG
    assert b"multiple of num_kv_heads" in lib.pa_last_error()


def test_decode_empty_batch_is_noop():
    lib, _ = _lib()
    assert _decode(lib, S=0, out=0, q=0, k=0, v=0, tables=0, lens=0) == 0


def _prefill(lib, **over):
    args = dict(out=16, q=32, k=48, v=64, tables=80, lens=96, qs=112, scale=0.1, bs=16, S=2, T=40, Hq=8, Hkv=2,
                D=128, NB=10, maxblk=4, maxq=32, maxctx=64, dtype=1, stream=None)
    args.update(over)
    return lib.pa_prefill(args["out"], args["q"], args["k"], args["v"], args["tables"], args["lens"], args["qs"],
                          args["scale"], args["bs"], args["S"], args["T"], args["Hq"], args["Hkv"], args["D"],
                          args["NB"], args["maxblk"], args["maxq"], args["maxctx"], args["dtype"], args["stream"])


@pytest.mark.parametrize("over,status,msg", [
    (dict(Hq=7), 1, b"multiple of num_kv_heads"),
    (dict(Hq=64, Hkv=2), 2, b"no prefill kernel"),   # group 32
    (dict(dtype=0, Hq=64, Hkv=2), 2, b"no prefill kernel"),  # float32 group 32
    (dict(D=96), 2, b"no prefill kernel"),
    (dict(bs=12), 2, b"power of two"),
    (dict(bs=512), 2, b"power of two"),
    (dict(T=-1), 1, b"zero size"),
    (dict(maxq=-1), 1, b"zero size"),
    (dict(maxblk=3), 1, b"max_blocks_per_seq"),
    (dict(dtype=7), 1, b"unknown dtype"),
    (dict(qs=0), 1, b"null pointer"),
    (dict(out=8), 1, b"16-byte aligned"),
    (dict(out=32), 1, b"aliases"),
    (dict(scale=float("nan")), 1, b"scale"),
])
def test_prefill_rejects_before_launch(over, status, msg):
    lib, _ = _lib()
    assert _prefill(lib, **over) == status
    assert msg in lib.pa_last_error()


def test_prefill_empty_is_noop():
    lib, _ = _lib()
    assert _prefill(lib, S=0, out=0, q=0, k=0, v=0, tables=0, lens=0, qs=0) == 0
    assert _prefill(lib, maxq=0, out=0, q=0, k=0, v=0, tables=0, lens=0, qs=0) == 0


def test_write_and_copy_reject_before_launch():
    lib, _ = _lib()
    assert lib.pa_write_cache(16, 16, 16, 16, 16, -1, 2, 128, 16, 10, 1, None) == 1
    assert lib.pa_write_cache(16, 16, 16, 16, 0, 3, 2, 128, 16, 10, 1, None) == 1
    assert lib.pa_write_cache(16, 16, 16, 16, 16, 3, 2, 4, 16, 10, 1, None) == 2  # 8-byte rows
    assert lib.pa_write_cache(0, 0, 0, 0, 0, 0, 2, 128, 16, 10, 1, None) == 0     # no tokens
    assert lib.pa_write_cache(16, 16, 16, 16, 16, 3, 2, 8200, 16, 10, 0, None) == 2  # 32800-byte rows
    assert b"32768" in lib.pa_last_error()
    assert lib.pa_copy_blocks(16, 16, 16, -2, 2, 16, 128, 10, 1, None) == 1
    assert lib.pa_copy_blocks(16, 16, 0, 2, 2, 16, 128, 10, 1, None) == 1
    assert lib.pa_copy_blocks(0, 0, 0, 0, 2, 16, 128, 10, 1, None) == 0
    assert lib.pa_copy_blocks(16, 16, 16, 2, 2, 16, 128, 10, 9, None) == 1


def test_layered_write_and_copy_reject_before_launch():
    lib, _ = _lib()
    assert lib.pa_write_cache_layers(16, 16, 16, 16, 16, 3, -1, 2, 128, 16, 10, 1, None) == 1
    assert lib.pa_write_cache_layers(16, 16, 16, 16, 16, 3, 70000, 2, 128, 16, 10, 1, None) == 2
    assert b"65535" in lib.pa_last_error()
    assert lib.pa_write_cache_layers(0, 0, 0, 0, 0, 3, 0, 2, 128, 16, 10, 1, None) == 0  # no layers
    assert lib.pa_write_cache_layers(16, 16, 16, 16, 16, 3, 2, 2, 4, 16, 10, 1, None) == 2  # 8-byte rows
    assert lib.pa_copy_blocks_layers(16, 16, 16, 2, -3, 2, 16, 128, 10, 1, None) == 1
    assert lib.pa_copy_blocks_layers(0, 0, 0, 2, 0, 2, 16, 128, 10, 1, None) == 0
    assert lib.pa_copy_blocks_layers(16, 16, 0, 2, 2, 2, 16, 128, 10, 1, None) == 1
    assert lib.pa_copy_blocks_layers(16, 16, 16, 2, 2, 2, 12, 128, 10, 1, None) == 2


def test_binding_refuses_cpu_tensors():
    _lib()
    import torch
    import paged_kv_cache_165_amd as pa
    q = torch.zeros(1, 4, 64)
    with pytest.raises(ValueError, match="GPU"):
        pa.decode(q.clone(), q, torch.zeros(2, 4, 16, 64), torch.zeros(2, 4, 16, 64),
                  torch.zeros(1, 1, dtype=torch.int32), torch.ones(1, dtype=torch.int32), 0.1, 1)


def test_missing_library_fails_loudly(tmp_path):
    from paged_kv_cache_165_amd import _lib as L
    with pytest.raises(L.LibraryNotBuilt):
        # a fresh loader pointed at a path that does not exist
        saved = L._lib
        L._lib = None
        try:
            L.load(str(tmp_path / "libpa.so"))
        finally:
            L._lib = saved


@pytest.mark.parametrize("args,status,msg", [
    ((16, 4, 32, 48, -1, 16), 1, b"zero size"),
    ((16, 0, 32, 48, 2, 16), 1, b"zero size"),
    ((16, 4, 32, 48, 2, 12), 2, b"power of two"),
    ((16, 4, 32, 48, 2, 512), 2, b"power of two"),
    ((0, 4, 32, 48, 2, 16), 1, b"null pointer"),
])
def test_append_block_tables_rejects_before_launch(args, status, msg):
    lib, _ = _lib()
    assert lib.pa_append_block_tables(*args, None) == status
    assert msg in lib.pa_last_error()
    assert lib.pa_append_block_tables(0, 4, 0, 0, 0, 16, None) == 0   # empty batch: nothing to do


@pytest.mark.parametrize("args,status,msg", [
    ((16, 4, 32, 48, 64, 80, -1, 16), 1, b"zero size"),
    ((16, 0, 32, 48, 64, 80, 2, 16), 1, b"zero size"),
    ((16, 4, 32, 48, 64, 80, 2, 12), 2, b"power of two"),
    ((16, 4, 32, 48, 64, 80, 2, 512), 2, b"power of two"),
    ((0, 4, 32, 48, 64, 80, 2, 16), 1, b"null pointer"),
    ((16, 4, 0, 48, 64, 80, 2, 16), 1, b"null pointer"),
    ((16, 4, 32, 0, 64, 80, 2, 16), 1, b"null pointer"),
    ((16, 4, 32, 48, 0, 80, 2, 16), 1, b"null pointer"),
    ((16, 4, 32, 48, 64, 0, 2, 16), 1, b"null pointer"),
])
def test_append_block_tables_host_rejects_before_launch(args, status, msg):
    """The host-argument append checks its arguments like the device one;
    the pointer values here are never dereferenced (the call fails first)."""
    lib, _ = _lib()
    assert lib.pa_append_block_tables_host(*args, None) == status
    assert msg in lib.pa_last_error()
    assert lib.pa_append_block_tables_host(0, 4, 0, 0, 0, 0, 0, 16, None) == 0   # empty batch: nothing to do



# (k, v, k_cache, v_cache, block_tables, max_blocks, host_lens, host_slots, lens_out, slots_out,
#  num_seqs, num_kv_heads, head_dim, block_size, num_blocks, dtype)
_WS = (16, 32, 48, 64, 80, 4, 96, 112, 128, 144, 2, 2, 128, 16, 10, 1)


def _ws(**kw):
    names = ("k", "v", "kc", "vc", "tab", "maxb", "lens", "slots", "lens_out", "slots_out", "n", "hkv", "d", "bs",
             "nb", "dt")
    a = dict(zip(names, _WS))
    a.update(kw)
    return tuple(a[n] for n in names)


@pytest.mark.parametrize("args,status,msg", [
    (_ws(n=-1), 1, b"zero size"),
    (_ws(maxb=0), 1, b"zero size"),
    (_ws(d=0), 1, b"zero size"),
    (_ws(nb=0), 1, b"zero size"),
    (_ws(dt=7), 1, b"unknown dtype"),
    (_ws(d=4), 2, b"multiple of 16"),
    (_ws(d=16384, dt=0), 2, b"more than 32768"),
    (_ws(bs=12), 2, b"power of two"),
    (_ws(bs=2), 2, b"power of two"),
    (_ws(bs=512), 2, b"power of two"),
    (_ws(k=0), 1, b"null pointer"),
    (_ws(tab=0), 1, b"null pointer"),
    (_ws(lens=0), 1, b"null pointer"),
    (_ws(slots_out=0), 1, b"null pointer"),
    (_ws(v=40), 1, b"aligned"),
    (_ws(kc=8), 1, b"aligned"),
])
def test_write_cache_append_host_rejects_before_launch(args, status, msg):
    """The append-and-write call checks its arguments before anything is
    launched; the pointer values here are never dereferenced."""
    lib, _ = _lib()
    assert lib.pa_write_cache_append_host(*args, None) == status
    assert msg in lib.pa_last_error()
    assert lib.pa_write_cache_append_host(*_ws(k=0, v=0, kc=0, vc=0, tab=0, n=0), None) == 0  # empty batch


def test_headers_and_library_usable_from_plain_c(tmp_path):
    """include/pa.h and include/pa_blocks.h compile as strict C99 (and as
    C++17), and a C program linked against libpa.so drives the host-side
    calls: version, status strings, the default partition, rejection before
    any launch, and the block manager's copy-on-write append
    (tests/c/abi_from_c.c)."""
    import shutil
    import subprocess
    from paged_kv_cache_165_amd import _lib as L
    gcc, gxx = shutil.which("gcc"), shutil.which("g++")
    if gcc is None or gxx is None:
        pytest.skip("no host C compiler")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    inc = os.path.join(root, "include")
    src = os.path.join(root, "tests", "c", "abi_from_c.c")
    libdir = os.path.dirname(L.LIB_PATH)
    strict = ["-Wall", "-Wextra", "-pedantic", "-Werror", f"-I{inc}"]
    subprocess.run([gxx, "-std=c++17", *strict, "-x", "c++", "-c", src, "-o", str(tmp_path / "cxx.o")], check=True)
    exe = str(tmp_path / "abi_from_c")
    subprocess.run([gcc, "-std=c99", *strict, src, f"-L{libdir}", "-lpa", f"-Wl,-rpath,{libdir}", "-o", exe],
                   check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stderr


def test_status_constants_match_header():
    """The binding's status codes are the header's enum values."""
    from paged_kv_cache_165_amd import _lib as L
    src = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "pa.h")).read()
    for name in ("PA_OK", "PA_ERR_INVALID_ARG", "PA_ERR_UNSUPPORTED", "PA_ERR_WORKSPACE", "PA_ERR_HIP",
                 "PA_ERR_NO_BLOCKS"):
        m = re.search(rf"\b{name}\s*=\s*(\d+)", src)
        assert m and int(m.group(1)) == getattr(L, name), name


def test_probe_rejects_before_launch():
    lib, L = _lib()
    p = ctypes.c_void_p(16)  # aligned, never dereferenced: every case fails on the host
    odd = ctypes.c_void_p(18)
    cases = [
        ((p, p, p, -1, 64, 4096, 2, 256, p), L.PA_ERR_INVALID_ARG),
        ((p, p, p, 4, 0, 4096, 2, 256, p), L.PA_ERR_INVALID_ARG),
        ((p, p, p, 4, 64, 4096, 2, 0, p), L.PA_ERR_INVALID_ARG),
        ((p, p, p, 4, 64, 3000, 2, 256, p), L.PA_ERR_UNSUPPORTED),
        ((p, p, p, 4, 64, 16384, 2, 256, p), L.PA_ERR_UNSUPPORTED),
        ((p, p, p, 4, 64, 4096, 3, 256, p), L.PA_ERR_UNSUPPORTED),
        ((None, p, p, 4, 64, 4096, 2, 256, p), L.PA_ERR_INVALID_ARG),
        ((odd, p, p, 4, 64, 4096, 2, 256, p), L.PA_ERR_INVALID_ARG),
    ]
    for args, status in cases:
        assert lib.pa_probe_read_tiles(*args, None) == status, args
    assert lib.pa_probe_read_tiles(None, None, None, 0, 64, 4096, 2, 256, None, None) == 0  # empty list: no-op
