"""Float64 CPU oracle for paged GQA decode attention — TEST INFRASTRUCTURE.

Only the test suite, the package smoke check and the bench's CPU-baseline leg
may import this package.  The GPU library never does, and this package imports
nothing from the GPU library.

  paged_attention(wl)      float64 [S, Hq, D]   (oracle.c)
  partials(wl, P, NP)      float64 m, l [S, Hq, NP], o [S, Hq, NP, D]
  merge(m, l, o, ...)      float64 [S, Hq, D]
  paged_varlen_arrays(...) float64 [total_q, Hq, D]: several causal query
                           tokens per sequence (oracle.c)
  plan(...)                the partition planner rule (planner.py)

Inputs are the numpy arrays of a `Workload` (fp16 pools, int32 tables).
`Oracle(path)` binds the same functions to another build of oracle.c (the
mutation tests compile deliberately broken copies and check that the pins
catch them).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from .planner import plan, PlanError  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "oracle.c")


def compile_oracle(src: str, out: str) -> str:
    """gcc, float64, no fast-math, no FMA contraction."""
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-pthread", src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    if force or not os.path.exists(LIB_PATH):
        compile_oracle(SRC_PATH, LIB_PATH)
    return LIB_PATH


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


class Oracle:
    """ctypes binding of one build of oracle.c."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32 = ctypes.c_int
        lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_half_to_double.restype = ctypes.c_double
        lib.oracle_paged_attention.argtypes = [P, P, P, P, P, i32, i32, i32, i32, i32, i32,
                                               ctypes.c_longlong, ctypes.c_double, P, i32]
        lib.oracle_paged_attention.restype = i32
        lib.oracle_partials.argtypes = [P, P, P, P, P, i32, i32, i32, i32, i32, i32,
                                        ctypes.c_longlong, ctypes.c_double, i32, i32, P, P, P,
                                        i32]
        lib.oracle_partials.restype = i32
        lib.oracle_merge.argtypes = [P, P, P, P, i32, i32, i32, i32, i32, P]
        lib.oracle_merge.restype = None
        lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_double.restype = ctypes.c_double
        lib.oracle_paged_attention_dt.argtypes = [P, P, P, P, P, i32, i32, i32, i32, i32, i32,
                                                  ctypes.c_longlong, ctypes.c_double, i32, P, i32]
        lib.oracle_paged_attention_dt.restype = i32
        lib.oracle_partials_dt.argtypes = [P, P, P, P, P, i32, i32, i32, i32, i32, i32,
                                           ctypes.c_longlong, ctypes.c_double, i32, i32, i32, P,
                                           P, P, i32]
        lib.oracle_partials_dt.restype = i32
        lib.oracle_paged_varlen.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, i32, i32,
                                            ctypes.c_longlong, ctypes.c_double, P, i32]
        lib.oracle_paged_varlen.restype = i32
        lib.oracle_paged_varlen_dt.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, i32, i32,
                                               ctypes.c_longlong, ctypes.c_double, i32, P, i32]
        lib.oracle_paged_varlen_dt.restype = i32
        self.lib = lib
        self.path = path

    def half_to_double(self, bits: int) -> float:
        return self.lib.oracle_half_to_double(int(bits) & 0xFFFF)

    def bf16_to_double(self, bits: int) -> float:
        return self.lib.oracle_bf16_to_double(int(bits) & 0xFFFF)

    # element type of q / K / V: numpy storage and the oracle's code
    DTYPES = {"f16": (np.float16, 0), "bf16": (np.uint16, 1), "f32": (np.float32, 2)}

    @classmethod
    def _args(cls, q, k_cache, v_cache, block_tables, seq_lens, dtype="f16"):
        st = cls.DTYPES[dtype][0]
        return (_c(q, st), _c(k_cache, st), _c(v_cache, st),
                _c(block_tables, np.int32), _c(seq_lens, np.int32))

    def paged_attention_arrays(self, q, k_cache, v_cache, block_tables, seq_lens, scale,
                               nthreads: int | None = None, dtype: str = "f16") -> np.ndarray:
        """dtype of q, K, V: "f16" (float16 arrays), "bf16" (uint16 bit
        patterns) or "f32" (float32 arrays)."""
        q, k, v, bt, sl = self._args(q, k_cache, v_cache, block_tables, seq_lens, dtype)
        S, Hq, D = q.shape
        nb, Hkv, bs, D2 = k.shape
        assert D2 == D and v.shape == k.shape and bt.shape[0] == S and sl.shape == (S,)
        out = np.empty((S, Hq, D), dtype=np.float64)
        st = self.lib.oracle_paged_attention_dt(_ptr(q), _ptr(k), _ptr(v), _ptr(bt), _ptr(sl), S,
                                                Hq, Hkv, D, bs, bt.shape[1], nb, float(scale),
                                                self.DTYPES[dtype][1], _ptr(out),
                                                nthreads or default_threads())
        if st != 0:
            raise ValueError(f"oracle_paged_attention failed: {st}")
        return out

    def paged_varlen_arrays(self, q, k_cache, v_cache, block_tables, seq_lens, cu_q, scale,
                            nthreads: int | None = None, dtype: str = "f16") -> np.ndarray:
        """Causal attention of packed query rows q [total_q, Hq, D] (sequence s
        owns rows cu_q[s] .. cu_q[s+1]-1, the last qlen_s of its L_s tokens);
        dtype of q, K, V as for paged_attention_arrays."""
        q, k, v, bt, sl = self._args(q, k_cache, v_cache, block_tables, seq_lens, dtype)
        cu = _c(cu_q, np.int32)
        T, Hq, D = q.shape
        nb, Hkv, bs, D2 = k.shape
        S = sl.shape[0]
        assert D2 == D and v.shape == k.shape and bt.shape[0] == S and cu.shape == (S + 1,)
        assert int(cu[0]) == 0 and int(cu[-1]) == T and np.all(np.diff(cu) >= 0)
        out = np.empty((T, Hq, D), dtype=np.float64)
        st = self.lib.oracle_paged_varlen_dt(_ptr(q), _ptr(k), _ptr(v), _ptr(bt), _ptr(sl),
                                             _ptr(cu), S, Hq, Hkv, D, bs, bt.shape[1], nb,
                                             float(scale), self.DTYPES[dtype][1], _ptr(out),
                                             nthreads or default_threads())
        if st != 0:
            raise ValueError(f"oracle_paged_varlen failed: {st}")
        return out

    def partials_arrays(self, q, k_cache, v_cache, block_tables, seq_lens, scale, P: int,
                        NP: int | None = None, nthreads: int | None = None, dtype: str = "f16"):
        q, k, v, bt, sl = self._args(q, k_cache, v_cache, block_tables, seq_lens, dtype)
        S, Hq, D = q.shape
        nb, Hkv, bs, _ = k.shape
        if NP is None:
            NP = max(1, -(-int(sl.max()) // P))
        m = np.full((S, Hq, NP), np.nan)
        l = np.full((S, Hq, NP), np.nan)
        o = np.full((S, Hq, NP, D), np.nan)
        st = self.lib.oracle_partials_dt(_ptr(q), _ptr(k), _ptr(v), _ptr(bt), _ptr(sl), S, Hq,
                                         Hkv, D, bs, bt.shape[1], nb, float(scale), int(P),
                                         int(NP), self.DTYPES[dtype][1], _ptr(m), _ptr(l),
                                         _ptr(o), nthreads or default_threads())
        if st != 0:
            raise ValueError(f"oracle_partials failed: {st}")
        return m, l, o

    def merge(self, m, l, o, seq_lens, P: int) -> np.ndarray:
        m = _c(m, np.float64)
        l = _c(l, np.float64)
        o = _c(o, np.float64)
        sl = _c(seq_lens, np.int32)
        S, Hq, NP, D = o.shape
        out = np.empty((S, Hq, D), dtype=np.float64)
        self.lib.oracle_merge(_ptr(m), _ptr(l), _ptr(o), _ptr(sl), S, Hq, D, int(P), NP,
                              _ptr(out))
        return out

    # Workload conveniences
    def paged_attention(self, wl, nthreads: int | None = None) -> np.ndarray:
        return self.paged_attention_arrays(wl.q, wl.k_cache, wl.v_cache, wl.block_tables,
                                           wl.seq_lens, wl.scale, nthreads,
                                           wl.meta.get("dtype", "f16"))

    def partials(self, wl, P: int, NP: int | None = None, nthreads: int | None = None):
        return self.partials_arrays(wl.q, wl.k_cache, wl.v_cache, wl.block_tables,
                                    wl.seq_lens, wl.scale, P, NP, nthreads,
                                    wl.meta.get("dtype", "f16"))


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        if not os.path.exists(LIB_PATH):
            build(force=False)
        _default = Oracle(LIB_PATH)
    return _default


def half_to_double(bits: int) -> float:
    return default().half_to_double(bits)


def paged_attention(wl, nthreads: int | None = None) -> np.ndarray:
    return default().paged_attention(wl, nthreads)


def paged_attention_arrays(*a, **kw) -> np.ndarray:
    return default().paged_attention_arrays(*a, **kw)


def partials(wl, P: int, NP: int | None = None, nthreads: int | None = None):
    return default().partials(wl, P, NP, nthreads)


def partials_arrays(*a, **kw):
    return default().partials_arrays(*a, **kw)


def paged_varlen_arrays(*a, **kw) -> np.ndarray:
    return default().paged_varlen_arrays(*a, **kw)


def merge(m, l, o, seq_lens, P: int) -> np.ndarray:
    return default().merge(m, l, o, seq_lens, P)
