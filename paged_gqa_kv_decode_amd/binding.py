"""ctypes binding of libvkpaged (include/vk_paged.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libvkpaged.so.  torch provides device memory (tensors) and the
stream handle.  If the library is not built, every call raises; there is no
CPU fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libvkpaged.so")

VK_OK = 0
STATUS_NAMES = {0: "OK", 1: "NULL_ARG", 2: "BAD_DIM", 3: "GEOMETRY", 4: "BLOCK_SIZE",
                5: "PARTITION", 6: "SEQ_LEN", 7: "SCRATCH_CAP", 8: "HIP", 9: "DTYPE",
                10: "ALIGN"}
DTYPE_F16, DTYPE_BF16, DTYPE_F32 = 0, 1, 2
KERNEL_AUTO, KERNEL_DOT, KERNEL_MFMA = 0, 1, 2
KERNEL_MFMA_W1, KERNEL_MFMA_W2, KERNEL_MFMA_W4, KERNEL_MFMA_W4P2 = 3, 4, 5, 6
KERNEL_VARLEN_COLUMNS, KERNEL_VARLEN_TILES = 7, 8
ORDER_AUTO, ORDER_GRID, ORDER_LONGEST_FIRST = 0, 1, 2

EXPORTED = ("vk_plan_partitions", "vk_paged_gqa_decode", "vk_paged_gqa_decode_fused",
            "vk_paged_gqa_reduce", "vk_paged_kv_append", "vk_select_decode_kernel",
            "vk_select_work_order", "vk_status_string", "vk_last_hip_error", "vk_trace_enabled",
            "vk_last_plan",
            "vk_plan_varlen", "vk_paged_gqa_varlen", "vk_paged_gqa_varlen_reduce",
            "vk_paged_gqa_decode_dt", "vk_select_varlen_kernel", "vk_paged_gqa_varlen_dt",
            "vk_paged_gqa_decode_noalloc")


class VkError(RuntimeError):
    def __init__(self, fn: str, code: int, detail: str = ""):
        name = STATUS_NAMES.get(code, str(code))
        msg = f"{fn} failed: VK_ERR_{name} ({status_string(code)})"
        if detail:
            msg += f" {detail}"
        super().__init__(msg)
        self.code = code
        self.name = name


class _Plan(ctypes.Structure):
    _fields_ = [("partition_size", ctypes.c_int32), ("max_num_partitions", ctypes.c_int32),
                ("work_full_parts", ctypes.c_int64), ("budget", ctypes.c_int64),
                ("cu_count", ctypes.c_int32), ("kernel", ctypes.c_int32),
                ("scratch_bytes", ctypes.c_uint64), ("grid", ctypes.c_int32 * 3),
                ("block", ctypes.c_int32), ("work_order", ctypes.c_int32)]


@dataclass
class Plan:
    partition_size: int
    max_num_partitions: int
    work_full_parts: int
    budget: int
    cu_count: int
    kernel: int
    scratch_bytes: int
    grid: tuple
    block: int
    work_order: int = 0

    @classmethod
    def from_c(cls, p: _Plan) -> "Plan":
        return cls(p.partition_size, p.max_num_partitions, p.work_full_parts, p.budget,
                   p.cu_count, p.kernel, p.scratch_bytes, tuple(p.grid), p.block, p.work_order)


_lib = None


def lib() -> ctypes.CDLL:
    """Load libvkpaged.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m paged_gqa_kv_decode_amd.build` (no CPU fallback exists)")
    # PyTorch ships its own HIP runtime.  Loading it first lets this library
    # bind to that same runtime (one per process); loaded the other way round
    # the process holds two, and this library's HIP calls found no device.
    import torch  # noqa: F401
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, u64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64
    L.vk_plan_partitions.argtypes = [vp, i32, i32, i32, i32, i32, i32, i32, i32, i32, u64,
                                     ctypes.POINTER(_Plan)]
    L.vk_plan_partitions.restype = i32
    L.vk_paged_gqa_decode.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i64,
                                      ctypes.c_float, i32, i32, vp, vp, vp, vp, vp]
    L.vk_paged_gqa_decode.restype = i32
    L.vk_paged_gqa_decode_dt.argtypes = [i32, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                         i64, ctypes.c_float, i32, i32, vp, vp, vp, vp, vp]
    L.vk_paged_gqa_decode_dt.restype = i32
    L.vk_paged_gqa_decode_fused.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                            i64, ctypes.c_float, i32, i32, vp, vp, vp, vp, vp, vp]
    L.vk_paged_gqa_decode_fused.restype = i32
    L.vk_paged_gqa_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                              i64, ctypes.c_float, i32, i32, vp, vp]
    L.vk_paged_gqa_decode_noalloc.restype = i32
    L.vk_plan_varlen.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, u64,
                                 ctypes.POINTER(_Plan)]
    L.vk_plan_varlen.restype = i32
    L.vk_paged_gqa_varlen.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                      i32, i64, ctypes.c_float, i32, i32, vp, vp, vp, vp, vp]
    L.vk_paged_gqa_varlen.restype = i32
    L.vk_paged_gqa_varlen_dt.argtypes = [i32] + L.vk_paged_gqa_varlen.argtypes
    L.vk_paged_gqa_varlen_dt.restype = i32
    L.vk_paged_gqa_varlen_reduce.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                             vp, vp]
    L.vk_paged_gqa_varlen_reduce.restype = i32
    L.vk_paged_gqa_reduce.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, vp]
    L.vk_paged_gqa_reduce.restype = i32
    L.vk_paged_kv_append.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i64,
                                     ctypes.c_double, vp, vp, vp]
    L.vk_paged_kv_append.restype = i32
    L.vk_select_decode_kernel.argtypes = [i32]
    L.vk_select_decode_kernel.restype = i32
    L.vk_select_work_order.argtypes = [i32]
    L.vk_select_work_order.restype = i32
    L.vk_select_varlen_kernel.argtypes = [i32]
    L.vk_select_varlen_kernel.restype = i32
    L.vk_status_string.argtypes = [i32]
    L.vk_status_string.restype = ctypes.c_char_p
    L.vk_last_hip_error.argtypes = []
    L.vk_last_hip_error.restype = i32
    L.vk_trace_enabled.argtypes = []
    L.vk_trace_enabled.restype = i32
    L.vk_last_plan.argtypes = [ctypes.POINTER(_Plan)]
    L.vk_last_plan.restype = i32
    _lib = L
    return L


def status_string(code: int) -> str:
    return lib().vk_status_string(int(code)).decode()


def _check(fn: str, code: int):
    if code != VK_OK:
        detail = ""
        if code == 8:
            detail = f"hip error {lib().vk_last_hip_error()}"
        raise VkError(fn, code, detail)


def select_decode_kernel(kernel: int) -> int:
    prev = lib().vk_select_decode_kernel(int(kernel))
    if prev < 0:
        raise ValueError(f"unknown decode kernel {kernel}")
    return prev


def select_work_order(order: int) -> int:
    prev = lib().vk_select_work_order(int(order))
    if prev < 0:
        raise ValueError(f"unknown work order {order}")
    return prev


def select_varlen_kernel(kernel: int) -> int:
    prev = lib().vk_select_varlen_kernel(int(kernel))
    if prev < 0:
        raise ValueError(f"unknown varlen kernel {kernel}")
    return prev


def last_plan() -> Plan:
    p = _Plan()
    _check("vk_last_plan", lib().vk_last_plan(ctypes.byref(p)))
    return Plan.from_c(p)


def plan_partitions(seq_lens_host, num_q_heads: int, num_kv_heads: int, head_dim: int,
                    block_size: int, max_blocks_per_seq: int, partition_request: int = -1,
                    cu_count: int = 0, budget_per_cu: int = 0,
                    scratch_cap_bytes: int = 0) -> Plan:
    sl = np.ascontiguousarray(np.asarray(seq_lens_host, dtype=np.int32))
    p = _Plan()
    code = lib().vk_plan_partitions(sl.ctypes.data if sl.size else None, int(sl.size),
                                    num_q_heads, num_kv_heads, head_dim, block_size,
                                    max_blocks_per_seq, partition_request, cu_count,
                                    budget_per_cu, scratch_cap_bytes, ctypes.byref(p))
    _check("vk_plan_partitions", code)
    return Plan.from_c(p)


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream_handle(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _need(t, dtype, name):
    import torch
    if t is None:
        return
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise TypeError(f"{name} must be a device tensor")
    _ = torch


def _torch_elem(dtype: int):
    import torch
    return {DTYPE_F16: torch.float16, DTYPE_BF16: torch.bfloat16, DTYPE_F32: torch.float32}[dtype]


def _decode_args(q, k_cache, v_cache, block_tables, seq_lens, scale, partition_size,
                 max_num_partitions, out, max_logits, exp_sums, tmp_out, dtype=DTYPE_F16):
    import torch
    et = _torch_elem(dtype)
    for t, dt, n in ((q, et, "q"), (k_cache, et, "k_cache"),
                     (v_cache, et, "v_cache"), (block_tables, torch.int32, "block_tables"),
                     (seq_lens, torch.int32, "seq_lens"), (out, torch.float32, "out"),
                     (max_logits, torch.float32, "max_logits"), (exp_sums, torch.float32, "exp_sums"),
                     (tmp_out, torch.float32, "tmp_out")):
        _need(t, dt, n)
    S, Hq, D = q.shape
    nb, Hkv, bs, D2 = k_cache.shape
    if D2 != D or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("k_cache / v_cache / q shapes disagree")
    if tuple(block_tables.shape[:1]) != (S,) or tuple(seq_lens.shape) != (S,):
        raise ValueError("block_tables / seq_lens must have num_seqs rows")
    if out is not None and tuple(out.shape) != (S, Hq, D):
        raise ValueError("out must be [S, Hq, D]")
    if partition_size:
        for t, shp, n in ((max_logits, (S, Hq, max_num_partitions), "max_logits"),
                          (exp_sums, (S, Hq, max_num_partitions), "exp_sums"),
                          (tmp_out, (S, Hq, max_num_partitions, D), "tmp_out")):
            if t is not None and tuple(t.shape) != shp:
                raise ValueError(f"{n} must be {shp}")
    return (_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(seq_lens), S, Hq, Hkv,
            D, bs, block_tables.shape[1], nb, float(scale), int(partition_size),
            int(max_num_partitions), _ptr(out), _ptr(max_logits), _ptr(exp_sums), _ptr(tmp_out))


def paged_gqa_decode(q, k_cache, v_cache, block_tables, seq_lens, scale: float,
                     partition_size: int, max_num_partitions: int, out=None, max_logits=None,
                     exp_sums=None, tmp_out=None, stream=None) -> None:
    """Enqueue the decode kernel.  Shapes are read from the tensors:
    q [S,Hq,D] fp16, k/v [num_blocks,Hkv,bs,D] fp16, block_tables [S,max_blocks]
    int32, seq_lens [S] int32; out [S,Hq,D] fp32 (unsplit) or max_logits /
    exp_sums [S,Hq,NP], tmp_out [S,Hq,NP,D] fp32 (split)."""
    args = _decode_args(q, k_cache, v_cache, block_tables, seq_lens, scale, partition_size,
                        max_num_partitions, out, max_logits, exp_sums, tmp_out)
    _check("vk_paged_gqa_decode", lib().vk_paged_gqa_decode(*args, _stream_handle(stream)))


def paged_gqa_decode_dt(dtype: int, q, k_cache, v_cache, block_tables, seq_lens, scale: float,
                        partition_size: int, max_num_partitions: int, out=None, max_logits=None,
                        exp_sums=None, tmp_out=None, stream=None) -> None:
    """paged_gqa_decode for q / K / V of element type `dtype` (DTYPE_F16,
    DTYPE_BF16 with torch.bfloat16 tensors, DTYPE_F32 with float32)."""
    args = _decode_args(q, k_cache, v_cache, block_tables, seq_lens, scale, partition_size,
                        max_num_partitions, out, max_logits, exp_sums, tmp_out, dtype)
    _check("vk_paged_gqa_decode_dt",
           lib().vk_paged_gqa_decode_dt(int(dtype), *args, _stream_handle(stream)))


def paged_gqa_decode_fused(q, k_cache, v_cache, block_tables, seq_lens, scale: float,
                           partition_size: int, max_num_partitions: int, out, max_logits=None,
                           exp_sums=None, tmp_out=None, counters=None, stream=None) -> None:
    """Enqueue decode + in-place merge as one launch: the final out [S,Hq,D]
    fp32 for any partition size.  Split calls also need the scratch of
    paged_gqa_decode and counters [S*Hkv] int32/uint32, zero before the first
    call (each call leaves it zero)."""
    import torch
    if out is None:
        raise ValueError("out is required")
    if partition_size:
        if counters is None or counters.dtype not in (torch.int32, torch.uint32) or \
                counters.device.type != "cuda":
            raise TypeError("counters must be a device int32/uint32 tensor")
        if counters.numel() < q.shape[0] * k_cache.shape[1]:
            raise ValueError("counters needs num_seqs * num_kv_heads entries")
    args = _decode_args(q, k_cache, v_cache, block_tables, seq_lens, scale, partition_size,
                        max_num_partitions, out, max_logits, exp_sums, tmp_out)
    _check("vk_paged_gqa_decode_fused",
           lib().vk_paged_gqa_decode_fused(*args, _ptr(counters) if partition_size else None,
                                           _stream_handle(stream)))


def paged_gqa_decode_noalloc(q, k_cache, v_cache, block_tables, seq_lens, scale: float,
                             partition_size: int, max_num_partitions: int, out,
                             stream=None) -> None:
    """Enqueue decode + reduce into out [S,Hq,D] fp32 with the split partials
    in the library's own device array (no scratch arguments; calls on one GPU
    must not overlap in time)."""
    if out is None:
        raise ValueError("out is required")
    args = _decode_args(q, k_cache, v_cache, block_tables, seq_lens, scale, partition_size,
                        max_num_partitions, out, None, None, None)
    _check("vk_paged_gqa_decode_noalloc",
           lib().vk_paged_gqa_decode_noalloc(*args[:16], _stream_handle(stream)))


def paged_gqa_reduce(max_logits, exp_sums, tmp_out, seq_lens, partition_size: int, out,
                     stream=None) -> None:
    """Enqueue the partition reduce: out [S,Hq,D] fp32 from the split partials."""
    import torch
    for t, dt, n in ((max_logits, torch.float32, "max_logits"), (exp_sums, torch.float32, "exp_sums"),
                     (tmp_out, torch.float32, "tmp_out"), (seq_lens, torch.int32, "seq_lens"),
                     (out, torch.float32, "out")):
        _need(t, dt, n)
    S, Hq, NP, D = tmp_out.shape
    if tuple(max_logits.shape) != (S, Hq, NP) or tuple(exp_sums.shape) != (S, Hq, NP):
        raise ValueError("partials shapes disagree")
    if tuple(out.shape) != (S, Hq, D) or tuple(seq_lens.shape) != (S,):
        raise ValueError("out / seq_lens shapes disagree")
    code = lib().vk_paged_gqa_reduce(_ptr(max_logits), _ptr(exp_sums), _ptr(tmp_out),
                                     _ptr(seq_lens), S, Hq, D, int(partition_size), NP,
                                     _ptr(out), _stream_handle(stream))
    _check("vk_paged_gqa_reduce", code)


def plan_varlen(seq_lens_host, q_lens_host, num_q_heads: int, num_kv_heads: int, head_dim: int,
                block_size: int, max_blocks_per_seq: int, partition_request: int = -1,
                cu_count: int = 0, scratch_cap_bytes: int = 0) -> Plan:
    sl = np.ascontiguousarray(np.asarray(seq_lens_host, dtype=np.int32))
    ql = np.ascontiguousarray(np.asarray(q_lens_host, dtype=np.int32))
    if sl.shape != ql.shape:
        raise ValueError("seq_lens and q_lens must have one entry per sequence")
    p = _Plan()
    code = lib().vk_plan_varlen(sl.ctypes.data if sl.size else None,
                                ql.ctypes.data if ql.size else None, int(sl.size), num_q_heads,
                                num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                                partition_request, cu_count, scratch_cap_bytes, ctypes.byref(p))
    _check("vk_plan_varlen", code)
    return Plan.from_c(p)


def paged_gqa_varlen(q, k_cache, v_cache, block_tables, seq_lens, cu_seqlens_q, max_q_len: int,
                     scale: float, partition_size: int, max_num_partitions: int, out=None,
                     max_logits=None, exp_sums=None, tmp_out=None, stream=None) -> None:
    """Enqueue the multi-token (causal, packed rows) kernel: q [total_q,Hq,D]
    fp16 or bf16 (K/V the same type), cu_seqlens_q [S+1] int32; out
    [total_q,Hq,D] fp32 (unsplit) or the partials [total_q,Hq,NP(,D)] (split)."""
    import torch
    et = torch.bfloat16 if q.dtype == torch.bfloat16 else torch.float16
    dtype = DTYPE_BF16 if et == torch.bfloat16 else DTYPE_F16
    for t, dt, n in ((q, et, "q"), (k_cache, et, "k_cache"),
                     (v_cache, et, "v_cache"), (block_tables, torch.int32, "block_tables"),
                     (seq_lens, torch.int32, "seq_lens"), (cu_seqlens_q, torch.int32, "cu_seqlens_q"),
                     (out, torch.float32, "out"), (max_logits, torch.float32, "max_logits"),
                     (exp_sums, torch.float32, "exp_sums"), (tmp_out, torch.float32, "tmp_out")):
        _need(t, dt, n)
    T, Hq, D = q.shape
    nb, Hkv, bs, D2 = k_cache.shape
    S = seq_lens.shape[0]
    if D2 != D or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("k_cache / v_cache / q shapes disagree")
    if block_tables.shape[0] != S or tuple(cu_seqlens_q.shape) != (S + 1,):
        raise ValueError("block_tables / cu_seqlens_q must match seq_lens")
    if out is not None and tuple(out.shape) != (T, Hq, D):
        raise ValueError("out must be [total_q, Hq, D]")
    if partition_size:
        for t, shp, n in ((max_logits, (T, Hq, max_num_partitions), "max_logits"),
                          (exp_sums, (T, Hq, max_num_partitions), "exp_sums"),
                          (tmp_out, (T, Hq, max_num_partitions, D), "tmp_out")):
            if t is not None and tuple(t.shape) != shp:
                raise ValueError(f"{n} must be {shp}")
    code = lib().vk_paged_gqa_varlen_dt(
        dtype, _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(seq_lens),
        _ptr(cu_seqlens_q), S, T, int(max_q_len), Hq, Hkv, D, bs, block_tables.shape[1], nb,
        float(scale), int(partition_size), int(max_num_partitions), _ptr(out), _ptr(max_logits),
        _ptr(exp_sums), _ptr(tmp_out), _stream_handle(stream))
    _check("vk_paged_gqa_varlen_dt", code)


def paged_gqa_varlen_reduce(max_logits, exp_sums, tmp_out, seq_lens, cu_seqlens_q,
                            max_q_len: int, partition_size: int, out, stream=None) -> None:
    """Enqueue the merge of the multi-token partials into out [total_q,Hq,D]."""
    import torch
    for t, dt, n in ((max_logits, torch.float32, "max_logits"), (exp_sums, torch.float32, "exp_sums"),
                     (tmp_out, torch.float32, "tmp_out"), (seq_lens, torch.int32, "seq_lens"),
                     (cu_seqlens_q, torch.int32, "cu_seqlens_q"), (out, torch.float32, "out")):
        _need(t, dt, n)
    T, Hq, NP, D = tmp_out.shape
    S = seq_lens.shape[0]
    if tuple(max_logits.shape) != (T, Hq, NP) or tuple(exp_sums.shape) != (T, Hq, NP):
        raise ValueError("partials shapes disagree")
    if tuple(out.shape) != (T, Hq, D) or tuple(cu_seqlens_q.shape) != (S + 1,):
        raise ValueError("out / cu_seqlens_q shapes disagree")
    code = lib().vk_paged_gqa_varlen_reduce(_ptr(max_logits), _ptr(exp_sums), _ptr(tmp_out),
                                            _ptr(seq_lens), _ptr(cu_seqlens_q), S, int(max_q_len),
                                            Hq, D, int(partition_size), NP, _ptr(out),
                                            _stream_handle(stream))
    _check("vk_paged_gqa_varlen_reduce", code)


class VarlenStep:
    """One multi-token step on device-resident inputs: plan once from the host
    lengths, hold the scratch, `run()` enqueues the kernel (+ reduce if split)."""

    def __init__(self, q, k_cache, v_cache, block_tables, seq_lens, cu_seqlens_q, seq_lens_host,
                 q_lens_host, scale: float, partition_request: int = -1, cu_count: int = 0,
                 out=None):
        import torch
        T, Hq, D = q.shape
        nb, Hkv, bs, _ = k_cache.shape
        self.plan = plan_varlen(seq_lens_host, q_lens_host, Hq, Hkv, D, bs, block_tables.shape[1],
                                partition_request, cu_count)
        self.max_q_len = int(max(1, int(np.max(q_lens_host))))
        self.args = (q, k_cache, v_cache, block_tables, seq_lens, cu_seqlens_q)
        self.scale = float(scale)
        dev = q.device
        self.out = out if out is not None else torch.empty((T, Hq, D), dtype=torch.float32,
                                                           device=dev)
        P, NP = self.plan.partition_size, self.plan.max_num_partitions
        if P:
            self.max_logits = torch.empty((T, Hq, NP), dtype=torch.float32, device=dev)
            self.exp_sums = torch.empty((T, Hq, NP), dtype=torch.float32, device=dev)
            self.tmp_out = torch.empty((T, Hq, NP, D), dtype=torch.float32, device=dev)
        else:
            self.max_logits = self.exp_sums = self.tmp_out = None

    def run(self, stream=None):
        P, NP = self.plan.partition_size, self.plan.max_num_partitions
        q, k, v, bt, sl, cu = self.args
        if P:
            paged_gqa_varlen(q, k, v, bt, sl, cu, self.max_q_len, self.scale, P, NP, None,
                             self.max_logits, self.exp_sums, self.tmp_out, stream)
            paged_gqa_varlen_reduce(self.max_logits, self.exp_sums, self.tmp_out, sl, cu,
                                    self.max_q_len, P, self.out, stream)
        else:
            paged_gqa_varlen(q, k, v, bt, sl, cu, self.max_q_len, self.scale, 0, 1, self.out,
                             stream=stream)
        return self.out


def paged_kv_append(k_new, v_new, block_tables, positions, k_cache, v_cache,
                    rope_theta: float = 0.0, stream=None) -> None:
    """Enqueue the append: k_new / v_new [S,Hkv,D] fp16, positions [S] int32,
    written into k_cache / v_cache [num_blocks,Hkv,bs,D] in place."""
    import torch
    for t, dt, n in ((k_new, torch.float16, "k_new"), (v_new, torch.float16, "v_new"),
                     (block_tables, torch.int32, "block_tables"), (positions, torch.int32, "positions"),
                     (k_cache, torch.float16, "k_cache"), (v_cache, torch.float16, "v_cache")):
        _need(t, dt, n)
    S, Hkv, D = k_new.shape
    nb, Hkv2, bs, D2 = k_cache.shape
    if tuple(v_new.shape) != (S, Hkv, D) or (Hkv2, D2) != (Hkv, D) or \
            tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("k_new / v_new / cache shapes disagree")
    if block_tables.shape[0] != S or tuple(positions.shape) != (S,):
        raise ValueError("block_tables / positions must have num_seqs rows")
    code = lib().vk_paged_kv_append(_ptr(k_new), _ptr(v_new), _ptr(block_tables), _ptr(positions),
                                    S, Hkv, D, bs, block_tables.shape[1], nb, float(rope_theta),
                                    _ptr(k_cache), _ptr(v_cache), _stream_handle(stream))
    _check("vk_paged_kv_append", code)


class DecodeStep:
    """One decode step on device-resident inputs: plan once (host seq_lens),
    hold the scratch, then `run()` enqueues decode (+ reduce when split), or
    the single-launch form when `fused`."""

    def __init__(self, q, k_cache, v_cache, block_tables, seq_lens, seq_lens_host, scale: float,
                 partition_request: int = -1, cu_count: int = 0, out=None, fused: bool = False,
                 dtype: int = DTYPE_F16):
        import torch
        S, Hq, D = q.shape
        nb, Hkv, bs, _ = k_cache.shape
        self.plan = plan_partitions(seq_lens_host, Hq, Hkv, D, bs, block_tables.shape[1],
                                    partition_request, cu_count)
        self.args = (q, k_cache, v_cache, block_tables, seq_lens)
        self.scale = float(scale)
        dev = q.device
        self.out = out if out is not None else torch.empty((S, Hq, D), dtype=torch.float32,
                                                           device=dev)
        P, NP = self.plan.partition_size, self.plan.max_num_partitions
        if P:
            self.max_logits = torch.empty((S, Hq, NP), dtype=torch.float32, device=dev)
            self.exp_sums = torch.empty((S, Hq, NP), dtype=torch.float32, device=dev)
            self.tmp_out = torch.empty((S, Hq, NP, D), dtype=torch.float32, device=dev)
        else:
            self.max_logits = self.exp_sums = self.tmp_out = None
        self.fused = bool(fused)
        self.dtype = int(dtype)
        # arrival counters of the single-launch form: zeroed once, every call
        # leaves them zero
        self.counters = (torch.zeros(S * Hkv, dtype=torch.int32, device=dev)
                         if (self.fused and P) else None)

    def run(self, stream=None):
        P, NP = self.plan.partition_size, self.plan.max_num_partitions
        q, k, v, bt, sl = self.args
        if self.fused:
            paged_gqa_decode_fused(q, k, v, bt, sl, self.scale, P, NP, self.out, self.max_logits,
                                   self.exp_sums, self.tmp_out, self.counters, stream)
        elif self.dtype != DTYPE_F16:
            paged_gqa_decode_dt(self.dtype, q, k, v, bt, sl, self.scale, P, NP,
                                None if P else self.out, self.max_logits, self.exp_sums,
                                self.tmp_out, stream)
            if P:
                paged_gqa_reduce(self.max_logits, self.exp_sums, self.tmp_out, sl, P, self.out,
                                 stream)
        elif P:
            paged_gqa_decode(q, k, v, bt, sl, self.scale, P, NP, None, self.max_logits,
                             self.exp_sums, self.tmp_out, stream)
            paged_gqa_reduce(self.max_logits, self.exp_sums, self.tmp_out, sl, P, self.out,
                             stream)
        else:
            paged_gqa_decode(q, k, v, bt, sl, self.scale, 0, 1, self.out, stream=stream)
        return self.out


def device_inputs(wl, device="cuda"):
    """Copy a Workload's host arrays to device tensors (q, k, v, bt, sl);
    bf16 workloads (uint16 bit patterns) become torch.bfloat16 tensors."""
    import torch
    dev = torch.device(device)

    def elem(a):
        t = torch.from_numpy(a)
        if wl.meta.get("dtype", "f16") == "bf16":
            t = t.view(torch.int16).view(torch.bfloat16)
        return t.to(dev)

    return (elem(wl.q), elem(wl.k_cache), elem(wl.v_cache),
            torch.from_numpy(wl.block_tables).to(dev), torch.from_numpy(wl.seq_lens).to(dev))
