"""Fused row-wise gated activations for AMD MI355X (gfx950).

A thin Python binding over libga.so (include/ga.h): it checks tensor shapes,
dtypes and contiguity, and passes device pointers, sizes and the current HIP
stream through the C-ABI.  Every step of the computation runs in the HIP
kernels; PyTorch only supplies device memory and the stream.  If the library
is not built, importing this package raises: there is no fallback.

    gelu_and_mul_sparse(x, z)           x: [T, 2d] -> [T, d] (round_intermediates=True:
                                        the round-trip form)
    gelu_and_mul_sparse_noalloc(x, z)   the same for T <= 256 rows, no workspace
                                        (the library's own static array)
    gelu_and_mul_sparse_down(x, w)      x: [T, 2d], w: [H, d] -> [T, H]: the activation
                                        fused with the down projection (bf16 / fp16)
    silu_and_mul_bounded(x, live_rows)  x: [M, 2d] -> [M, d] (live rows only)
    gelu_and_mul(x, approximate)        x: [T, 2d] -> [T, d] (tanh or erf GELU)
    squared_relu_bounded(x, live_rows)  x: [M, d]  -> [M, d] (live rows only)
    z_from_sparsity(p)                  Phi^-1(p), host-side
"""
from ._lib import (  # noqa: F401
    GA_BF16, GA_F16, GA_F32, GA_OK, GA_EINVAL, GA_EUNSUPPORTED, GA_EHIP, GA_MAX_D, GA_ROUND_INTERMEDIATES,
    GaError, Plan, Z_SPARSITY_095, lib, library_path,
    gelu_and_mul_sparse, gelu_and_mul_sparse_noalloc, silu_and_mul_bounded, stream_xor_rows,
    gelu_and_mul, squared_relu_bounded, z_from_sparsity,
    plan_gelu_and_mul_sparse, plan_silu_and_mul_bounded, workspace_for,
    reserve_workspace, held_workspaces, GA_SPLIT_PLAN_ROWS, WORKSPACE_BYTES,
    DownPlan, GA_DOWN_MAX_ROWS, GA_DOWN_DECODE, GA_DOWN_STAGED, GA_DOWN_TILED,
    gelu_and_mul_sparse_down, plan_gelu_and_mul_sparse_down,
    gelu_and_mul_sparse_down_workspace_bytes, reserve_down_workspace,
)
