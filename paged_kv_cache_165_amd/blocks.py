"""Host-side block manager: a thin wrapper over the native one declared in
include/pa_blocks.h (argument marshalling only; the bookkeeping runs in
libpa.so)."""

from __future__ import annotations

import ctypes

import numpy as np

from . import _lib

PA_ERR_INVALID_ARG = 1
PA_ERR_NO_BLOCKS = 5


class BlocksExhausted(RuntimeError):
    """Not enough free blocks; the manager is unchanged."""


def _check(lib, status: int) -> None:
    if status == 0:
        return
    msg = lib.pa_last_error().decode()
    if status == PA_ERR_NO_BLOCKS:
        raise BlocksExhausted(msg)
    raise ValueError(msg)


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


class BlockManager:
    """Block tables, reference counts and copy-on-write pairs of a pool of
    ``num_blocks`` blocks of ``block_size`` tokens (see include/pa_blocks.h).
    ``free_order`` lists every block id once in hand-out order (default
    0, 1, 2, ...). Sequence ids are Python ints (64-bit)."""

    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        self._lib = _lib.load()
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        handle = ctypes.c_void_p()
        order = None
        if free_order is not None:
            order = np.ascontiguousarray(np.asarray(free_order, dtype=np.int32))
            if order.shape != (self.num_blocks,):
                raise ValueError("free_order must list every block once")
        _check(self._lib, self._lib.pa_bm_create(self.num_blocks, self.block_size,
                                                 None if order is None else _ptr(order),
                                                 ctypes.byref(handle)))
        self._h = handle

    def close(self) -> None:
        if getattr(self, "_h", None):
            self._lib.pa_bm_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    # -- sequence operations ---------------------------------------------
    def prefill(self, seq: int, num_tokens: int) -> None:
        _check(self._lib, self._lib.pa_bm_prefill(self._h, int(seq), int(num_tokens)))

    def share(self, seq: int, src: int, num_tokens: int) -> None:
        _check(self._lib, self._lib.pa_bm_share(self._h, int(seq), int(src), int(num_tokens)))

    def append(self, seqs) -> tuple[np.ndarray, np.ndarray]:
        """Reserve the next slot of each sequence; returns (slots int32 [n],
        copy-on-write pairs int32 [k, 2])."""
        s = np.ascontiguousarray(np.asarray(seqs, dtype=np.int64))
        n = len(s)
        slots = np.empty(n, np.int32)
        pairs = np.empty((max(n, 1), 2), np.int32)
        k = ctypes.c_int(0)
        _check(self._lib, self._lib.pa_bm_append(self._h, _ptr(s), n, _ptr(slots), _ptr(pairs), ctypes.byref(k)))
        return slots, pairs[:k.value].copy()

    def append_into(self, seqs: np.ndarray, slots: np.ndarray, pairs: np.ndarray) -> int:
        """``append`` writing straight into caller arrays: ``seqs`` int64 [n],
        ``slots`` int32 [n], ``pairs`` int32 [>= n, 2] (C-contiguous);
        returns the number of copy pairs."""
        k = ctypes.c_int(0)
        _check(self._lib, self._lib.pa_bm_append(self._h, _ptr(seqs), len(seqs), _ptr(slots), _ptr(pairs),
                                                 ctypes.byref(k)))
        return k.value

    def block_tables_into(self, seqs: np.ndarray, tables: np.ndarray, lens: np.ndarray, pad: int = 0) -> None:
        """``block_tables`` writing straight into ``tables`` int32 [n, max_blocks]
        and ``lens`` int32 [n] (C-contiguous)."""
        _check(self._lib, self._lib.pa_bm_block_tables(self._h, _ptr(seqs), len(seqs), _ptr(tables),
                                                       tables.shape[1], int(pad), _ptr(lens)))

    def free(self, seq: int) -> None:
        _check(self._lib, self._lib.pa_bm_free(self._h, int(seq)))

    def block_tables(self, seqs, max_blocks: int, pad: int = 0) -> tuple[np.ndarray, np.ndarray]:
        """(tables int32 [n, max_blocks] padded with ``pad``, context lengths int32 [n])."""
        s = np.ascontiguousarray(np.asarray(seqs, dtype=np.int64))
        n = len(s)
        tables = np.empty((n, max_blocks), np.int32)
        lens = np.empty(n, np.int32)
        _check(self._lib, self._lib.pa_bm_block_tables(self._h, _ptr(s), n, _ptr(tables), int(max_blocks),
                                                       int(pad), _ptr(lens)))
        return tables, lens

    # -- accounting ---------------------------------------------------------
    def refcount(self, block: int) -> int:
        return int(self._lib.pa_bm_refcount(self._h, int(block)))

    def num_free(self) -> int:
        return int(self._lib.pa_bm_num_free(self._h))

    def blocks_in_use(self) -> int:
        return int(self._lib.pa_bm_blocks_in_use(self._h))

    def seq_tokens(self, seq: int) -> int:
        return int(self._lib.pa_bm_seq_tokens(self._h, int(seq)))

    def blocks_without_sharing(self) -> int:
        return int(self._lib.pa_bm_blocks_without_sharing(self._h))

    def check(self) -> None:
        _check(self._lib, self._lib.pa_bm_check(self._h))
