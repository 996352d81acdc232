"""gemm_block_bit_amd: fused dequantize-and-multiply GEMV/GEMM over weight-only
quantized LLM layers on AMD MI355X (gfx950).

The work is done by libgbb.so (C ABI in include/gbb.h: a host packer and HIP
kernels).  This package only marshals arguments: numpy arrays for the host
packer, torch tensors for device memory and the current HIP stream.  There is
no CPU fallback -- if the library is missing every call raises.
"""
from .binding import (  # noqa: F401
    Batched,
    GbbError,
    Graph,
    allocate_bits,
    channel_order,
    check_image,
    dequant,
    gemm_mixed_w,
    gemm_mixed_w_64x64,
    gemm_mixed_w_64x64_path,
    gemm_mixed_w_64x64_workspace,
    gemm_mixed_w_batched_workspace,
    gemm_mixed_w_noalloc,
    gemm_mixed_w_path,
    gemm_mixed_w_workspace,
    gemm_w48a8,
    gemm_w48a8_workspace,
    lib,
    pack_blocks,
    pack_w48,
    packed_bytes,
    quant_act_i8,
    unpack_codes,
    version,
    w48_group_acc,
    w48_packed_bytes,
)
