"""ctypes binding of the host block manager in libpa.so (include/pa_block_manager.h).

Argument marshalling only: every decision (which blocks, which slots, which
copies) is made by the native manager.  Host arrays are NumPy; the results
are what the device entry points take -- int64 slots for ``write_kv``,
``(src, dst)`` pairs for ``copy_blocks``, int32 table rows and context
lengths for the decode calls -- once the caller moves them to the GPU.
"""

from __future__ import annotations

import ctypes

import numpy as np

from .binding import PagedAttentionError, load_library

PA_OK = 0
PA_ERR_INVALID_ARG = -1
PA_ERR_NO_BLOCKS = -5
PA_ERR_STATE = -6

EXPORTED_BM = (
    "pa_bm_create", "pa_bm_destroy", "pa_bm_num_free_blocks", "pa_bm_ref_count",
    "pa_bm_context_len", "pa_bm_can_allocate", "pa_bm_allocate", "pa_bm_fork",
    "pa_bm_blocks_needed_to_append", "pa_bm_append", "pa_bm_free", "pa_bm_block_tables",
)

_declared = False


def _lib():
    global _declared
    lib = load_library()
    if not _declared:
        P, I = ctypes.c_void_p, ctypes.c_int32
        sig = {
            "pa_bm_create": (ctypes.c_int, [I, I, I, I, P, ctypes.POINTER(P)]),
            "pa_bm_destroy": (None, [P]),
            "pa_bm_num_free_blocks": (I, [P]),
            "pa_bm_ref_count": (I, [P, I]),
            "pa_bm_context_len": (I, [P, I]),
            "pa_bm_can_allocate": (ctypes.c_int, [P, I]),
            "pa_bm_allocate": (ctypes.c_int, [P, I, I, P]),
            "pa_bm_fork": (ctypes.c_int, [P, I, I]),
            "pa_bm_blocks_needed_to_append": (ctypes.c_int, [P, P, I]),
            "pa_bm_append": (ctypes.c_int, [P, P, I, P, P, P]),
            "pa_bm_free": (ctypes.c_int, [P, I]),
            "pa_bm_block_tables": (ctypes.c_int, [P, P, I, P, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _declared = True
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data if a.size else None


class BlockManager:
    """Handle on a native block manager; statuses are returned, not raised,
    except by the constructor."""

    def __init__(self, num_blocks: int, block_size: int, max_seqs: int, max_blocks_per_seq: int,
                 free_order=None):
        self._lib = _lib()
        self.num_blocks, self.block_size = int(num_blocks), int(block_size)
        self.max_seqs, self.max_blocks = int(max_seqs), int(max_blocks_per_seq)
        order = None
        if free_order is not None:
            order = np.ascontiguousarray(free_order, dtype=np.int32)
            if order.shape != (self.num_blocks,):
                raise PagedAttentionError("free_order must hold num_blocks ids")
        h = ctypes.c_void_p()
        st = self._lib.pa_bm_create(self.num_blocks, self.block_size, self.max_seqs,
                                    self.max_blocks, None if order is None else _ptr(order),
                                    ctypes.byref(h))
        if st != PA_OK:
            raise PagedAttentionError(f"pa_bm_create: status {st}")
        self._h = h
        self._slots = np.empty(self.max_seqs, dtype=np.int64)
        self._pairs = np.empty((self.max_seqs, 2), dtype=np.int64)

    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value:
            self._lib.pa_bm_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        self.close()

    # ---- queries
    def num_free(self) -> int:
        return int(self._lib.pa_bm_num_free_blocks(self._h))

    def ref_count(self, block: int) -> int:
        return int(self._lib.pa_bm_ref_count(self._h, int(block)))

    def context_len(self, seq: int) -> int:
        return int(self._lib.pa_bm_context_len(self._h, int(seq)))

    def can_allocate(self, num_tokens: int) -> bool:
        st = self._lib.pa_bm_can_allocate(self._h, int(num_tokens))
        if st < 0:
            raise PagedAttentionError(f"pa_bm_can_allocate: status {st}")
        return st == 1

    # ---- operations
    def allocate(self, seq: int, num_tokens: int):
        slots = np.empty(max(int(num_tokens), 0), dtype=np.int64)
        st = self._lib.pa_bm_allocate(self._h, int(seq), int(num_tokens), _ptr(slots))
        return st, (slots if st == PA_OK else np.empty(0, dtype=np.int64))

    def fork(self, parent: int, child: int) -> int:
        return self._lib.pa_bm_fork(self._h, int(parent), int(child))

    def blocks_needed_to_append(self, seqs) -> int:
        s = np.ascontiguousarray(seqs, dtype=np.int32)
        return self._lib.pa_bm_blocks_needed_to_append(self._h, _ptr(s), int(s.size))

    def append(self, seqs):
        """Returns (status, int64 slots [n], list of (src, dst) copy pairs)."""
        s = np.ascontiguousarray(seqs, dtype=np.int32)
        n = int(s.size)
        if n > self.max_seqs:        # cannot be distinct sequences
            return PA_ERR_INVALID_ARG, np.empty(0, dtype=np.int64), []
        ncopy = ctypes.c_int32(0)
        st = self._lib.pa_bm_append(self._h, _ptr(s), n, self._slots.ctypes.data,
                                    self._pairs.ctypes.data, ctypes.byref(ncopy))
        if st != PA_OK:
            return st, np.empty(0, dtype=np.int64), []
        k = int(ncopy.value)
        return st, self._slots[:n].copy(), [(int(a), int(b)) for a, b in self._pairs[:k]]

    def free_seq(self, seq: int) -> int:
        return self._lib.pa_bm_free(self._h, int(seq))

    def block_tables(self, seqs=None):
        """int32 rows [n, max_blocks_per_seq] padded with -1, int32 lengths [n]
        (rows 0..max_seqs-1 when ``seqs`` is None)."""
        if seqs is None:
            n, sp = self.max_seqs, None
        else:
            s = np.ascontiguousarray(seqs, dtype=np.int32)
            n, sp = int(s.size), _ptr(s)
        rows = np.empty((n, self.max_blocks), dtype=np.int32)
        lens = np.empty(n, dtype=np.int32)
        st = self._lib.pa_bm_block_tables(self._h, sp, n, _ptr(rows), _ptr(lens))
        if st != PA_OK:
            raise PagedAttentionError(f"pa_bm_block_tables: status {st}")
        return rows, lens
