"""Python face of the plain fp64 CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product library or its binding.
It shares no code with the GPU path; both sides only consume the seeded inputs
of the `workloads` package.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "oracle.c")
LIB = os.path.join(_HERE, "liboracle.so")

FMT = {"bf16": 0, "fp8": 1, "mxfp8": 2, "mxfp4": 3}
WFMT = {"f32": 0, "bf16": 1}
GCC_FLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-shared", "-fPIC"]


def compile_source(src: str, out: str) -> str:
    """gcc -O2 -fopenmp (no fast-math, no contraction) `src` into shared library `out`."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *GCC_FLAGS, src, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        compile_source(SRC, LIB)
    return LIB


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


class Oracle:
    """ctypes binding of one compiled oracle library."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        lib.oracle_windows.argtypes = [ctypes.c_int] * 3 + [P] * 5
        lib.oracle_windows.restype = None
        lib.oracle_windows_thd.argtypes = [ctypes.c_int, P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P]
        lib.oracle_windows_thd.restype = None
        lib.oracle_gather_paged.argtypes = [ctypes.c_int] * 4 + [P] * 4 + [ctypes.c_int] * 2 + [P] * 2
        lib.oracle_gather_paged.restype = None
        lib.oracle_windows_paged.argtypes = [ctypes.c_int] * 3 + [P] * 3
        lib.oracle_windows_paged.restype = None
        lib.oracle_mqa_logits.argtypes = ([ctypes.c_int] * 6 + [P] * 5 + [ctypes.c_int, ctypes.c_double]
                                          + [P, P, P, ctypes.c_int64, P, P, ctypes.c_int])
        lib.oracle_mqa_logits.restype = ctypes.c_int
        lib.oracle_topk.argtypes = [ctypes.c_int64, ctypes.c_int, P, ctypes.c_int64, P, P, ctypes.c_int, ctypes.c_int,
                                    P, P]
        lib.oracle_topk.restype = ctypes.c_int
        for name, argt in (("oracle_dec_bf16", ctypes.c_uint16), ("oracle_dec_e4m3", ctypes.c_uint8),
                           ("oracle_dec_e2m1", ctypes.c_uint8), ("oracle_dec_e8m0", ctypes.c_uint8)):
            fn = getattr(lib, name)
            fn.argtypes = [argt]
            fn.restype = ctypes.c_double
        self.lib = lib
        self.path = path

    def decode(self, fmt: str, code: int) -> float:
        """One element code -> its exact value (fmt in bf16, e4m3, e2m1, e8m0)."""
        return getattr(self.lib, "oracle_dec_" + fmt)(code)

    def windows_thd(self, cu_q, cu_k, ratio: int, T_q: int, m_total: int) -> tuple[np.ndarray, np.ndarray]:
        """Packed variable-length windows with ratio-compressed keys, int32 [T_q] arrays."""
        cq = np.ascontiguousarray(cu_q, np.int32)
        ck = np.ascontiguousarray(cu_k, np.int32)
        assert cq.size == ck.size and cq.size >= 2
        ws = np.empty(T_q, np.int32)
        we = np.empty(T_q, np.int32)
        self.lib.oracle_windows_thd(cq.size - 1, _ptr(cq), _ptr(ck), int(ratio), int(T_q), int(m_total), _ptr(ws),
                                    _ptr(we))
        return ws, we

    def gather_paged(self, wl):
        """The dense K ([B, S_k, row bytes] codes) and K scales of a paged workload."""
        pg = wl.paged
        cache = np.ascontiguousarray(pg["k_cache"])
        row_bytes = cache.dtype.itemsize * int(np.prod(cache.shape[2:]))
        scache = None if pg["k_scale_cache"] is None else np.ascontiguousarray(pg["k_scale_cache"])
        scale_bytes = 0 if scache is None else scache.dtype.itemsize
        k = np.empty((wl.B, wl.S_k) + cache.shape[2:], cache.dtype)
        ks = None if scache is None else np.empty((wl.B, wl.S_k), scache.dtype)
        bt = np.ascontiguousarray(pg["block_table"], np.int32)
        ctx = np.ascontiguousarray(pg["ctx"], np.int32)
        self.lib.oracle_gather_paged(wl.B, wl.S_k, row_bytes, scale_bytes, _ptr(cache), _ptr(scache), _ptr(bt),
                                     _ptr(ctx), int(pg["page_size"]), bt.shape[1], _ptr(k), _ptr(ks))
        return k, ks

    def dense(self, wl):
        """A paged workload with its K gathered (windows still from the context lengths)."""
        if getattr(wl, "paged", None) is None:
            return wl
        k, ks = self.gather_paged(wl)
        return wl.replace(k=k, k_scale=ks)

    def windows(self, wl) -> tuple[np.ndarray, np.ndarray]:
        """Per-row [start, end) of a workload as int32 [B, S_q] arrays."""
        if getattr(wl, "paged", None) is not None:
            ws = np.empty((wl.B, wl.S_q), np.int32)
            we = np.empty((wl.B, wl.S_q), np.int32)
            ctx = np.ascontiguousarray(wl.paged["ctx"], np.int32)
            self.lib.oracle_windows_paged(wl.B, wl.S_q, wl.S_k, _ptr(ctx), _ptr(ws), _ptr(we))
            return ws, we
        if getattr(wl, "thd", None) is not None:
            assert wl.B == 1
            ws, we = self.windows_thd(wl.thd["cu_q"], wl.thd["cu_k"], wl.thd["ratio"], wl.S_q, wl.S_k)
            return ws.reshape(1, -1), we.reshape(1, -1)
        ws = np.empty((wl.B, wl.S_q), np.int32)
        we = np.empty((wl.B, wl.S_q), np.int32)
        offs = None if wl.offsets is None else np.ascontiguousarray(wl.offsets, np.int32)
        st = None if wl.starts is None else np.ascontiguousarray(wl.starts, np.int32)
        en = None if wl.ends is None else np.ascontiguousarray(wl.ends, np.int32)
        self.lib.oracle_windows(wl.B, wl.S_q, wl.S_k, _ptr(offs), _ptr(st), _ptr(en), _ptr(ws), _ptr(we))
        return ws, we

    def topk(self, vals: np.ndarray, win_start: np.ndarray, win_end: np.ndarray, k: int, by_column: bool = False):
        """Top-k of every row of `vals` ([n_rows, >= S_k] fp32, or bf16 given as
        uint16 bits) inside its window: (idx int32 [n_rows, k], val fp32
        [n_rows, k]), in rank order or by ascending column.  win_start /
        win_end: [n_rows] int32, within [0, S_k]."""
        v = np.asarray(vals)
        if v.dtype == np.uint16:
            v = (v.astype(np.uint32) << 16).view(np.float32)
        v = np.ascontiguousarray(v, np.float32)
        assert v.ndim == 2
        ws = np.ascontiguousarray(np.asarray(win_start).reshape(-1), np.int32)
        we = np.ascontiguousarray(np.asarray(win_end).reshape(-1), np.int32)
        n_rows = v.shape[0]
        assert ws.size == n_rows and we.size == n_rows and k >= 1
        assert np.all(ws >= 0) and np.all(we <= v.shape[1])
        idx = np.empty((n_rows, k), np.int32)
        val = np.empty((n_rows, k), np.float32)
        if self.lib.oracle_topk(n_rows, v.shape[1], _ptr(v), v.shape[1], _ptr(ws), _ptr(we), int(k),
                                int(bool(by_column)), _ptr(idx), _ptr(val)) != 0:
            raise MemoryError("oracle_topk")
        return idx, val

    def logits(self, wl, rows: Optional[Sequence[int]] = None, threads: int = 0, return_threads: bool = False):
        """fp64 scores and per-cell error scales.

        rows: global row ids b*S_q+i to evaluate (None: all rows).  Returns
        (ref, bound) as float64 [n_rows, S_k] (and the thread count if asked)."""
        ws, we = self.windows(wl)
        wl = self.dense(wl)
        if rows is None:
            n_rows, rows_arr = wl.B * wl.S_q, None
        else:
            rows_arr = np.ascontiguousarray(np.asarray(rows, np.int64))
            n_rows = rows_arr.size
        ref = np.empty((n_rows, wl.S_k), np.float64)
        bound = np.empty((n_rows, wl.S_k), np.float64)
        arrs = [None if a is None else np.ascontiguousarray(a) for a in (wl.q, wl.q_scale, wl.k, wl.k_scale, wl.w)]
        used = self.lib.oracle_mqa_logits(wl.B, wl.S_q, wl.S_k, wl.H, wl.D, FMT[wl.fmt], *[_ptr(a) for a in arrs],
                                          WFMT[wl.w_dtype], float(wl.sm_scale), _ptr(ws), _ptr(we),
                                          _ptr(rows_arr), n_rows, _ptr(ref), _ptr(bound), int(threads))
        if used < 0:
            raise RuntimeError("oracle_mqa_logits rejected its arguments")
        return (ref, bound, used) if return_threads else (ref, bound)


_default: Optional[Oracle] = None


def default() -> Oracle:
    global _default
    if _default is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build(force=True)
        _default = Oracle(LIB)
    return _default


def decode(fmt: str, code: int) -> float:
    return default().decode(fmt, code)


def windows(wl):
    return default().windows(wl)


def windows_thd(cu_q, cu_k, ratio, T_q, m_total):
    return default().windows_thd(cu_q, cu_k, ratio, T_q, m_total)


def logits(wl, rows=None, threads: int = 0, return_threads: bool = False):
    return default().logits(wl, rows=rows, threads=threads, return_threads=return_threads)


def topk(vals, win_start, win_end, k, by_column=False):
    return default().topk(vals, win_start, win_end, k, by_column=by_column)
