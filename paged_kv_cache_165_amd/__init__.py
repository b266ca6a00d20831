"""Paged KV-cache decode attention for MI355X (gfx950).

Thin Python binding over the C ABI of ``libpa.so`` (include/pa.h). Every
function checks tensor devices, dtypes, shapes and contiguity, then passes raw
device pointers and the current torch stream to the library; all computation
runs in the library's HIP kernels. PyTorch supplies device memory and
streams only. There is no fallback path: a missing library raises.

Layouts (see include/pa.h):
  k_cache           [num_blocks, num_kv_heads, block_size, head_dim]
  v_cache           [num_blocks, num_kv_heads, block_size // T, head_dim, T],
                    T = min(block_size, 16) (``v_cache_shape``)
  q, out            [num_seqs, num_heads, head_dim]
                    (prefill: [num_tokens, num_heads, head_dim], split by query_start)
  query_start       int32 [num_seqs + 1] (prefill)
  k, v              [num_tokens, num_kv_heads, head_dim]
  block_tables      int32 [num_seqs, max_blocks_per_seq]
  context_lens      int32 [num_seqs]
  slot_mapping      int32 [num_tokens]
  src_dst_pairs     int32 [num_pairs, 2]
"""

from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

from . import _lib

__all__ = [
    "PaError", "library", "default_partition_size", "workspace_size", "alloc_workspace",
    "v_tile", "v_cache_shape", "alloc_cache",
    "decode", "decode_partitions", "decode_merge", "append_block_tables", "append_block_tables_host", "prefill", "write_cache", "copy_blocks",
    "alloc_cache_layers", "write_cache_layers", "copy_blocks_layers", "decode_plan", "probe_read_tiles",
    "debug_enabled", "check_slot_mapping", "check_copy_pairs", "check_decode_inputs", "decode_noalloc",
]

_DTYPES = {torch.float32: _lib.PA_F32, torch.bfloat16: _lib.PA_BF16, torch.float16: _lib.PA_F16}


class PaError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        super().__init__(f"pa status {status}: {message}")


def library() -> ctypes.CDLL:
    return _lib.load()


def _check(status: int) -> None:
    if status != _lib.PA_OK:
        lib = library()
        raise PaError(status, f"{lib.pa_status_string(status).decode()}: {lib.pa_last_error().decode()}")


def _dev_tensor(t: torch.Tensor, name: str, dtype=None, ndim=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU, got {t.device}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


# ---------------------------------------------------------------------------
# Debug precondition checks (PA_DEBUG=1)
# ---------------------------------------------------------------------------
#
# The kernels clamp what they read, so a bad index gives wrong values, never a
# fault; they cannot tell a caller that broke a precondition. With the
# environment variable PA_DEBUG=1 the binding copies the index arrays of each
# call to the host (a synchronizing copy: keep it off timed paths) and checks
# them first, the debug consistency check the cf-1.com blog describes (4.3).
# The checks are plain functions of host arrays and can be called directly.

def debug_enabled() -> bool:
    return os.environ.get("PA_DEBUG", "") == "1"


def _host_ints(a) -> np.ndarray:
    if isinstance(a, torch.Tensor):
        a = a.detach().to("cpu")
        return a.numpy()
    return np.asarray(a)


def check_slot_mapping(slot_mapping, num_blocks: int, block_size: int) -> None:
    """Every slot is -1 (skip) or in [0, num_blocks * block_size), and no two
    tokens name the same slot (pa_write_cache leaves either value there)."""
    s = _host_ints(slot_mapping).astype(np.int64).ravel()
    bad = s[(s < -1) | (s >= num_blocks * block_size)]
    if bad.size:
        raise ValueError(f"slot_mapping holds {bad.size} slot(s) outside {{-1}} and [0, {num_blocks * block_size}): "
                         f"{bad[:4].tolist()}")
    live = s[s >= 0]
    u, c = np.unique(live, return_counts=True)
    if (c > 1).any():
        raise ValueError(f"slot_mapping names slot(s) {u[c > 1][:4].tolist()} more than once")


def check_copy_pairs(src_dst_pairs, num_blocks: int) -> None:
    """Every id is in [0, num_blocks), every dst is distinct and no dst is
    also a src (pairs act as if applied at once)."""
    p = _host_ints(src_dst_pairs).astype(np.int64).reshape(-1, 2)
    bad = p[(p < 0) | (p >= num_blocks)]
    if bad.size:
        raise ValueError(f"src_dst_pairs holds block id(s) outside [0, {num_blocks}): {bad[:4].tolist()}")
    u, c = np.unique(p[:, 1], return_counts=True)
    if (c > 1).any():
        raise ValueError(f"src_dst_pairs copies into block(s) {u[c > 1][:4].tolist()} more than once")
    both = np.intersect1d(p[:, 0], p[:, 1])
    if both.size:
        raise ValueError(f"block(s) {both[:4].tolist()} are both a copy source and a copy destination")


def check_decode_inputs(block_tables, context_lens, num_blocks: int, block_size: int, max_context_len: int) -> None:
    """Every context length is in [0, max_context_len] and every table entry
    a sequence reads (the first ceil(L / B)) is a block of the pool."""
    t = _host_ints(block_tables).astype(np.int64)
    lens = _host_ints(context_lens).astype(np.int64).ravel()
    bad = np.nonzero((lens < 0) | (lens > max_context_len))[0]
    if bad.size:
        raise ValueError(f"context_lens of sequence(s) {bad[:4].tolist()} outside [0, {max_context_len}]")
    need = -(-lens // block_size)
    if t.ndim != 2 or (need > t.shape[1]).any():
        raise ValueError("a context needs more table entries than a row holds")
    cols = np.arange(t.shape[1])[None, :]
    read = cols < need[:, None]
    badt = read & ((t < 0) | (t >= num_blocks))
    if badt.any():
        s, j = np.argwhere(badt)[0]
        raise ValueError(f"block_tables[{s}][{j}] = {t[s, j]} is outside [0, {num_blocks}) and is read")


def _stream(t: torch.Tensor) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def v_tile(block_size: int) -> int:
    """Tokens per transposed V tile of the cache layout."""
    return min(block_size, 16)


def v_cache_shape(num_blocks: int, num_kv_heads: int, block_size: int, head_dim: int) -> tuple:
    t = v_tile(block_size)
    return (num_blocks, num_kv_heads, block_size // t, head_dim, t)


def alloc_cache(num_blocks: int, num_kv_heads: int, block_size: int, head_dim: int,
                dtype=torch.bfloat16, device="cuda"):
    """Uninitialised (k_cache, v_cache) pair in the library's layout."""
    k = torch.empty(num_blocks, num_kv_heads, block_size, head_dim, dtype=dtype, device=device)
    v = torch.empty(v_cache_shape(num_blocks, num_kv_heads, block_size, head_dim), dtype=dtype, device=device)
    return k, v


def _check_caches(k_cache, v_cache):
    _dev_tensor(k_cache, "k_cache", ndim=4)
    if k_cache.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {k_cache.dtype}")
    _dev_tensor(v_cache, "v_cache", dtype=k_cache.dtype, ndim=5)
    nb, hkv, bs, d = k_cache.shape
    if tuple(v_cache.shape) != v_cache_shape(nb, hkv, bs, d):
        raise ValueError(f"v_cache must have shape {v_cache_shape(nb, hkv, bs, d)} "
                         f"(transposed tiles), got {tuple(v_cache.shape)}")
    return nb, hkv, bs, d


def default_partition_size(num_seqs: int, num_heads: int, num_kv_heads: int, max_context_len: int,
                           block_size: int, dtype: torch.dtype) -> int:
    """Partition ``decode`` uses for ``partition_size=0`` on a batch of this shape."""
    return int(library().pa_default_partition_size(num_seqs, num_heads, num_kv_heads, max_context_len,
                                                   block_size, _DTYPES[dtype]))


def workspace_size(num_seqs: int, num_heads: int, num_kv_heads: int, head_dim: int, max_context_len: int,
                   block_size: int, partition_size: int, dtype: torch.dtype) -> int:
    return int(library().pa_decode_workspace_size(num_seqs, num_heads, num_kv_heads, head_dim,
                                                  max_context_len, block_size, partition_size, _DTYPES[dtype]))


def alloc_workspace(num_seqs: int, num_heads: int, num_kv_heads: int, head_dim: int, max_context_len: int,
                    block_size: int, partition_size: int, dtype: torch.dtype, device="cuda") -> torch.Tensor:
    """Caller-owned workspace tensor (uint8) for ``decode``."""
    n = workspace_size(num_seqs, num_heads, num_kv_heads, head_dim, max_context_len, block_size, partition_size,
                       dtype)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def _decode_args(out, q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len,
                 partition_size, workspace):
    _dev_tensor(q, "q", ndim=3)
    if q.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    _dev_tensor(out, "out", dtype=q.dtype, ndim=3)
    if k_cache.dtype != q.dtype:
        raise ValueError(f"k_cache must be {q.dtype}, got {k_cache.dtype}")
    nb, hkv, bs, d2 = _check_caches(k_cache, v_cache)
    _dev_tensor(block_tables, "block_tables", dtype=torch.int32, ndim=2)
    _dev_tensor(context_lens, "context_lens", dtype=torch.int32, ndim=1)
    s, hq, d = q.shape
    if tuple(out.shape) != (s, hq, d):
        raise ValueError("out must have the shape of q")
    if d2 != d:
        raise ValueError("cache head_dim differs from q")
    if block_tables.shape[0] != s or context_lens.shape[0] != s:
        raise ValueError("one block table row and one context length per sequence")
    if max_context_len is None:
        max_context_len = int(context_lens.max().item()) if s else 0  # device -> host read
    if debug_enabled():
        check_decode_inputs(block_tables, context_lens, nb, bs, int(max_context_len))
    if workspace is None:
        workspace = alloc_workspace(s, hq, hkv, d, max_context_len, bs, partition_size, q.dtype, device=q.device)
    else:
        _dev_tensor(workspace, "workspace")
    ws_bytes = workspace.numel() * workspace.element_size()
    return (out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
            block_tables.data_ptr(), context_lens.data_ptr(), float(scale), bs, s, hq, hkv, d, nb,
            block_tables.shape[1], int(max_context_len), int(partition_size), _DTYPES[q.dtype],
            workspace.data_ptr(), ws_bytes, _stream(q))


def decode(out, q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len=None,
           partition_size=0, workspace=None, shared_blocks=False):
    """Paged decode attention into ``out`` (see ``pa_decode`` in include/pa.h).

    ``max_context_len`` should be passed by callers that know it; when None it
    is read from the device, which synchronizes the stream. ``shared_blocks``
    is the hint that some physical blocks appear in several tables
    (``pa_decode_ex`` with PA_DECODE_SHARED_BLOCKS): the same results, read
    through the L2 for the other sharers.
    """
    args = _decode_args(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                        max_context_len, partition_size, workspace)
    if shared_blocks:
        _check(library().pa_decode_ex(*args[:-1], _lib.PA_DECODE_SHARED_BLOCKS, args[-1]))
    else:
        _check(library().pa_decode(*args))
    return out


def decode_noalloc(out, q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len: int,
                   partition_size: int = 0):
    """``decode`` without a workspace and without any allocation
    (``pa_decode_noalloc``): the split-K records go to the library's static
    device scratch of ``_lib.NOALLOC_SCRATCH_BYTES`` bytes per GPU. Calls that
    overlap on one GPU race. ``max_context_len`` is required (reading it from
    the device would synchronize)."""
    _dev_tensor(q, "q", ndim=3)
    if q.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    _dev_tensor(out, "out", dtype=q.dtype, ndim=3)
    if k_cache.dtype != q.dtype:
        raise ValueError(f"k_cache must be {q.dtype}, got {k_cache.dtype}")
    nb, hkv, bs, d2 = _check_caches(k_cache, v_cache)
    _dev_tensor(block_tables, "block_tables", dtype=torch.int32, ndim=2)
    _dev_tensor(context_lens, "context_lens", dtype=torch.int32, ndim=1)
    s, hq, d = q.shape
    if tuple(out.shape) != (s, hq, d) or d2 != d:
        raise ValueError("out must have the shape of q, the caches its head_dim")
    if block_tables.shape[0] != s or context_lens.shape[0] != s:
        raise ValueError("one block table row and one context length per sequence")
    if debug_enabled():
        check_decode_inputs(block_tables, context_lens, nb, bs, int(max_context_len))
    _check(library().pa_decode_noalloc(out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                       block_tables.data_ptr(), context_lens.data_ptr(), float(scale), bs, s, hq,
                                       hkv, d, nb, block_tables.shape[1], int(max_context_len), int(partition_size),
                                       _DTYPES[q.dtype], _stream(q)))
    return out


def decode_partitions(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                      max_context_len, partition_size=0, workspace=None, shared_blocks=False):
    """First stage of ``decode`` (partition kernel) on the current stream;
    ``shared_blocks`` as in ``decode``."""
    args = _decode_args(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                        max_context_len, partition_size, workspace)
    if shared_blocks:
        _check(library().pa_decode_partitions_ex(*args[:-1], _lib.PA_DECODE_SHARED_BLOCKS, args[-1]))
    else:
        _check(library().pa_decode_partitions(*args))


def decode_merge(out, q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len,
                 partition_size=0, workspace=None):
    """Second stage of ``decode`` (log-sum-exp merge) on the current stream."""
    args = _decode_args(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                        max_context_len, partition_size, workspace)
    _check(library().pa_decode_merge(*args))


def prefill(out, q, k_cache, v_cache, block_tables, context_lens, query_start, scale,
            max_query_len=None, max_context_len=None):
    """Paged prefill attention into ``out`` (see ``pa_prefill`` in include/pa.h):
    the new tokens of sequence s are rows query_start[s]:query_start[s + 1] of
    ``q``, the last of its context_lens[s] cached tokens, each attending to the
    tokens up to its own position.

    ``max_query_len`` and ``max_context_len`` should be passed by callers that
    know them; when None they are read from the device, which synchronizes the
    stream.
    """
    _dev_tensor(q, "q", ndim=3)
    if q.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {q.dtype}")
    _dev_tensor(out, "out", dtype=q.dtype, ndim=3)
    if k_cache.dtype != q.dtype:
        raise ValueError(f"k_cache must be {q.dtype}, got {k_cache.dtype}")
    nb, hkv, bs, d2 = _check_caches(k_cache, v_cache)
    _dev_tensor(block_tables, "block_tables", dtype=torch.int32, ndim=2)
    _dev_tensor(context_lens, "context_lens", dtype=torch.int32, ndim=1)
    _dev_tensor(query_start, "query_start", dtype=torch.int32, ndim=1)
    n, hq, d = q.shape
    s = context_lens.shape[0]
    if tuple(out.shape) != (n, hq, d):
        raise ValueError("out must have the shape of q")
    if d2 != d:
        raise ValueError("cache head_dim differs from q")
    if block_tables.shape[0] != s or query_start.shape[0] != s + 1:
        raise ValueError("one block table row and one context length per sequence, num_seqs + 1 query starts")
    if max_query_len is None:
        max_query_len = int((query_start[1:] - query_start[:-1]).max().item()) if s else 0
    if max_context_len is None:
        max_context_len = int(context_lens.max().item()) if s else 0
    if debug_enabled():
        check_decode_inputs(block_tables, context_lens, nb, bs, int(max_context_len))
    _check(library().pa_prefill(out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                block_tables.data_ptr(), context_lens.data_ptr(), query_start.data_ptr(),
                                float(scale), bs, s, n, hq, hkv, d, nb, block_tables.shape[1],
                                int(max_query_len), int(max_context_len), _DTYPES[q.dtype], _stream(q)))
    return out


def write_cache(k, v, k_cache, v_cache, slot_mapping):
    """Write new tokens' K/V rows into their slots (``pa_write_cache``)."""
    nb, hkv, bs, d = _check_caches(k_cache, v_cache)
    _dev_tensor(k, "k", dtype=k_cache.dtype, ndim=3)
    _dev_tensor(v, "v", dtype=k_cache.dtype, ndim=3)
    _dev_tensor(slot_mapping, "slot_mapping", dtype=torch.int32, ndim=1)
    n = slot_mapping.shape[0]
    if tuple(k.shape) != (n, hkv, d) or tuple(v.shape) != (n, hkv, d):
        raise ValueError("k and v must be [num_tokens, num_kv_heads, head_dim]")
    if debug_enabled():
        check_slot_mapping(slot_mapping, nb, bs)
    _check(library().pa_write_cache(k.data_ptr(), v.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                    slot_mapping.data_ptr(), n, hkv, d, bs, nb, _DTYPES[k_cache.dtype],
                                    _stream(k_cache)))


def copy_blocks(k_cache, v_cache, src_dst_pairs):
    """Copy whole blocks src -> dst in both caches (``pa_copy_blocks``)."""
    nb, hkv, bs, d = _check_caches(k_cache, v_cache)
    _dev_tensor(src_dst_pairs, "src_dst_pairs", dtype=torch.int32, ndim=2)
    if src_dst_pairs.shape[1] != 2:
        raise ValueError("src_dst_pairs must be [num_pairs, 2]")
    if debug_enabled():
        check_copy_pairs(src_dst_pairs, nb)
    _check(library().pa_copy_blocks(k_cache.data_ptr(), v_cache.data_ptr(), src_dst_pairs.data_ptr(),
                                    src_dst_pairs.shape[0], hkv, bs, d, nb, _DTYPES[k_cache.dtype],
                                    _stream(k_cache)))


def append_block_tables(block_tables, context_lens, slot_mapping, block_size: int):
    """Record each sequence's newest block in its device table row
    (``pa_append_block_tables``): block_tables[i][(L - 1) // B] =
    slot_mapping[i] // B for L = context_lens[i] >= 1 and a slot >= 0."""
    _dev_tensor(block_tables, "block_tables", dtype=torch.int32, ndim=2)
    _dev_tensor(context_lens, "context_lens", dtype=torch.int32, ndim=1)
    _dev_tensor(slot_mapping, "slot_mapping", dtype=torch.int32, ndim=1)
    n = block_tables.shape[0]
    if context_lens.shape[0] != n or slot_mapping.shape[0] != n:
        raise ValueError("one context length and one slot per table row")
    _check(library().pa_append_block_tables(block_tables.data_ptr(), block_tables.shape[1], context_lens.data_ptr(),
                                            slot_mapping.data_ptr(), n, int(block_size), _stream(block_tables)))


def _host_int32(a, name: str) -> np.ndarray:
    if isinstance(a, torch.Tensor):
        if a.device.type != "cpu":
            raise ValueError(f"{name} must be in host memory")
        a = a.numpy()
    a = np.asarray(a)
    if a.dtype != np.int32 or a.ndim != 1:
        raise ValueError(f"{name} must be a 1-D int32 host array")
    return np.ascontiguousarray(a)


def append_block_tables_host(block_tables, context_lens, slot_mapping, context_lens_out, slot_mapping_out,
                             block_size: int):
    """``append_block_tables`` with the lengths and slots given as host int32
    arrays (``pa_append_block_tables_host``): they travel in the launch
    arguments, are stored to the device tensors ``context_lens_out`` and
    ``slot_mapping_out``, and the host arrays may be reused as soon as this
    returns."""
    _dev_tensor(block_tables, "block_tables", dtype=torch.int32, ndim=2)
    _dev_tensor(context_lens_out, "context_lens_out", dtype=torch.int32, ndim=1)
    _dev_tensor(slot_mapping_out, "slot_mapping_out", dtype=torch.int32, ndim=1)
    lens = _host_int32(context_lens, "context_lens")
    slots = _host_int32(slot_mapping, "slot_mapping")
    n = block_tables.shape[0]
    if lens.shape[0] != n or slots.shape[0] != n or context_lens_out.shape[0] != n or slot_mapping_out.shape[0] != n:
        raise ValueError("one context length and one slot per table row")
    _check(library().pa_append_block_tables_host(block_tables.data_ptr(), block_tables.shape[1],
                                                 lens.ctypes.data, slots.ctypes.data, context_lens_out.data_ptr(),
                                                 slot_mapping_out.data_ptr(), n, int(block_size),
                                                 _stream(block_tables)))


def write_cache_append_host(k, v, k_cache, v_cache, block_tables, context_lens, slot_mapping, context_lens_out,
                            slot_mapping_out):
    """``append_block_tables_host`` then ``write_cache`` of row i of ``k``/``v``
    ([num_seqs, num_kv_heads, head_dim]) into slot ``slot_mapping[i]``, in one
    launch per 448 sequences (``pa_write_cache_append_host``). The lengths and
    slots are host int32 arrays carried in the launch arguments."""
    nb, hkv, bs, d = _check_caches(k_cache, v_cache)
    _dev_tensor(k, "k", dtype=k_cache.dtype, ndim=3)
    _dev_tensor(v, "v", dtype=k_cache.dtype, ndim=3)
    _dev_tensor(block_tables, "block_tables", dtype=torch.int32, ndim=2)
    _dev_tensor(context_lens_out, "context_lens_out", dtype=torch.int32, ndim=1)
    _dev_tensor(slot_mapping_out, "slot_mapping_out", dtype=torch.int32, ndim=1)
    lens = _host_int32(context_lens, "context_lens")
    slots = _host_int32(slot_mapping, "slot_mapping")
    n = block_tables.shape[0]
    if lens.shape[0] != n or slots.shape[0] != n or context_lens_out.shape[0] != n or slot_mapping_out.shape[0] != n:
        raise ValueError("one context length and one slot per table row")
    if tuple(k.shape) != (n, hkv, d) or tuple(v.shape) != (n, hkv, d):
        raise ValueError("k and v must be [num_seqs, num_kv_heads, head_dim]")
    if debug_enabled():
        check_slot_mapping(slots, nb, bs)
    _check(library().pa_write_cache_append_host(k.data_ptr(), v.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                                block_tables.data_ptr(), block_tables.shape[1], lens.ctypes.data,
                                                slots.ctypes.data, context_lens_out.data_ptr(),
                                                slot_mapping_out.data_ptr(), n, hkv, d, bs, nb,
                                                _DTYPES[k_cache.dtype], _stream(k_cache)))


def alloc_cache_layers(num_layers: int, num_blocks: int, num_kv_heads: int, block_size: int, head_dim: int,
                       dtype=torch.bfloat16, device="cuda"):
    """Uninitialised (k_cache, v_cache) of ``num_layers`` layers in one
    allocation each: [L, NB, Hkv, B, D] and [L, *v_cache_shape]."""
    k = torch.empty(num_layers, num_blocks, num_kv_heads, block_size, head_dim, dtype=dtype, device=device)
    v = torch.empty(num_layers, *v_cache_shape(num_blocks, num_kv_heads, block_size, head_dim), dtype=dtype,
                    device=device)
    return k, v


def _check_layer_caches(k_cache, v_cache):
    _dev_tensor(k_cache, "k_cache", ndim=5)
    if k_cache.dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {k_cache.dtype}")
    _dev_tensor(v_cache, "v_cache", dtype=k_cache.dtype, ndim=6)
    nl, nb, hkv, bs, d = k_cache.shape
    if tuple(v_cache.shape) != (nl, *v_cache_shape(nb, hkv, bs, d)):
        raise ValueError(f"v_cache must have shape {(nl, *v_cache_shape(nb, hkv, bs, d))}, got {tuple(v_cache.shape)}")
    return nl, nb, hkv, bs, d


def write_cache_layers(k, v, k_cache, v_cache, slot_mapping):
    """``write_cache`` for every layer in one launch (``pa_write_cache_layers``):
    k, v [L, num_tokens, Hkv, D]; caches from ``alloc_cache_layers``."""
    nl, nb, hkv, bs, d = _check_layer_caches(k_cache, v_cache)
    _dev_tensor(k, "k", dtype=k_cache.dtype, ndim=4)
    _dev_tensor(v, "v", dtype=k_cache.dtype, ndim=4)
    _dev_tensor(slot_mapping, "slot_mapping", dtype=torch.int32, ndim=1)
    n = slot_mapping.shape[0]
    if tuple(k.shape) != (nl, n, hkv, d) or tuple(v.shape) != (nl, n, hkv, d):
        raise ValueError("k and v must be [num_layers, num_tokens, num_kv_heads, head_dim]")
    if debug_enabled():
        check_slot_mapping(slot_mapping, nb, bs)
    _check(library().pa_write_cache_layers(k.data_ptr(), v.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                           slot_mapping.data_ptr(), n, nl, hkv, d, bs, nb, _DTYPES[k_cache.dtype],
                                           _stream(k_cache)))


def copy_blocks_layers(k_cache, v_cache, src_dst_pairs):
    """``copy_blocks`` for every layer in one launch (``pa_copy_blocks_layers``)."""
    nl, nb, hkv, bs, d = _check_layer_caches(k_cache, v_cache)
    _dev_tensor(src_dst_pairs, "src_dst_pairs", dtype=torch.int32, ndim=2)
    if src_dst_pairs.shape[1] != 2:
        raise ValueError("src_dst_pairs must be [num_pairs, 2]")
    if debug_enabled():
        check_copy_pairs(src_dst_pairs, nb)
    _check(library().pa_copy_blocks_layers(k_cache.data_ptr(), v_cache.data_ptr(), src_dst_pairs.data_ptr(),
                                           src_dst_pairs.shape[0], nl, hkv, bs, d, nb, _DTYPES[k_cache.dtype],
                                           _stream(k_cache)))


def decode_plan(num_seqs: int, num_heads: int, num_kv_heads: int, head_dim: int, max_context_len: int,
                block_size: int, partition_size: int, dtype: torch.dtype, lds_per_cu: int = 163840,
                lds_per_workgroup: int = 163840, max_workgroups_per_cu: int = 1) -> dict:
    """The partition kernel, LDS request and result ring ``decode`` would use
    for this shape (``pa_decode_plan``, host only)."""
    plan = _lib.DecodePlan()
    _check(library().pa_decode_plan(num_seqs, num_heads, num_kv_heads, head_dim, max_context_len, block_size,
                                    partition_size, _DTYPES[dtype], lds_per_cu, lds_per_workgroup,
                                    max_workgroups_per_cu, ctypes.byref(plan)))
    names = {_lib.PA_DECODE_VALU: "valu", _lib.PA_DECODE_MFMA: "mfma", _lib.PA_DECODE_MFMA_WAVE: "mfma_wave",
             _lib.PA_DECODE_MFMA_STREAM: "mfma_stream"}
    return {"kernel": names[plan.kernel], "partition_size": plan.partition_size, "lds_bytes": plan.lds_bytes,
            "ring_slots": plan.ring_slots, "workgroups_per_cu": plan.workgroups_per_cu}


def probe_read_tiles(k_cache, v_cache, tiles, tiles_in_flight: int, workgroups: int, sink, tile_bytes=None):
    """Bandwidth probe (``pa_probe_read_tiles``, include/pa_probe.h): read the
    K and V tiles listed in ``tiles`` with the decode's loads and no
    arithmetic. A tile is ``tile_bytes`` of the cache (default: the whole
    (block, KV head) slice, block * head_dim elements) and ``tiles`` holds
    int32 tile indices. ``sink`` must hold 16 * 256 * workgroups bytes."""
    nb, hkv, bs, d = _check_caches(k_cache, v_cache)
    _dev_tensor(tiles, "tiles", dtype=torch.int32, ndim=1)
    _dev_tensor(sink, "sink")
    if sink.numel() * sink.element_size() < 16 * 256 * workgroups:
        raise ValueError("sink too small")
    slice_bytes = bs * d * k_cache.element_size()
    tile_bytes = slice_bytes if tile_bytes is None else int(tile_bytes)
    if tile_bytes <= 0 or slice_bytes % tile_bytes != 0:
        raise ValueError(f"tile_bytes {tile_bytes} must divide the (block, head) slice of {slice_bytes} bytes")
    _check(library().pa_probe_read_tiles(k_cache.data_ptr(), v_cache.data_ptr(), tiles.data_ptr(), tiles.shape[0],
                                         nb * hkv * (slice_bytes // tile_bytes), tile_bytes, int(tiles_in_flight),
                                         int(workgroups),
                                         sink.data_ptr(), _stream(k_cache)))
