"""MI355X-native FP8 (E4M3 / E5M2) block-scaled NT GEMM with BF16 output: dense,
contiguous grouped and masked grouped (MoE) forms, plus the fp8 block quantisation in
front of it.

The compute path is libdg.so (HIP kernels for gfx950 behind the C ABI in
include/dg.h); this package exposes the same call names through a thin ctypes binding.
"""
from .binding import (DG_CONTIGUOUS, DG_DENSE, DG_FP8_E4M3, DG_FP8_E5M2,  # noqa: F401
                      DG_MASKED, DGError, LIB_PATH, dg_gemm_fp8_nt,
                      dg_get_m_alignment_for_contiguous_layout,
                      dg_grouped_gemm_fp8_contiguous, dg_grouped_gemm_fp8_masked,
                      dg_instance_name, dg_quantize_fp8_128x128, dg_quantize_fp8_1x128,
                      dg_status_string, dg_transpose_fp8, dg_workspace_bytes, group_sizes_to_idx,
                      load_library)
