"""paged_gqa_kv_decode_amd — paged GQA decode attention for AMD MI355X.

The compute path is libvkpaged.so (HIP kernels for gfx950 behind a C ABI,
include/vk_paged.h); `binding` marshals torch tensors into it.  `workloads`
draws the seeded synthetic inputs.
"""
from .binding import (  # noqa: F401
    DecodeStep, KERNEL_AUTO, KERNEL_DOT, KERNEL_MFMA, KERNEL_MFMA_W1, KERNEL_MFMA_W2, KERNEL_MFMA_W4, KERNEL_MFMA_W4P2, Plan, VkError, device_inputs, last_plan,
    lib, paged_gqa_decode, paged_gqa_decode_dt, paged_gqa_decode_fused, DTYPE_F16, DTYPE_BF16,
    DTYPE_F32, paged_gqa_reduce, paged_kv_append,
    plan_partitions, plan_varlen, paged_gqa_varlen, paged_gqa_varlen_reduce, VarlenStep,
    select_decode_kernel, select_work_order, ORDER_AUTO, ORDER_GRID, ORDER_LONGEST_FIRST,
    status_string,
)
