"""MI355X (gfx950) MoE dispatch / combine: routing layout, BF16 / FP8 E4M3
dispatch, gate-weighted combine and their backward pair as hand-written HIP
kernels behind a C ABI
(include/ep.h, libep.so).  `ep` is the ctypes binding; `workloads` draws the
seeded synthetic inputs; `build` compiles the library in-tree."""
from .ep import (EP_BF16, EP_FP8_E4M3, EP_MXFP4_E2M1, EP_MXFP8_E4M3, EpError, EpShape, LayoutBuffers, Prepared, alloc_recv, ep_abi_version,
                 ep_check_cvt_bf16, ep_check_cvt_e2m1, ep_check_cvt_e4m3, ep_combine, ep_combine_backward,
                 ep_dispatch, ep_dispatch_backward, ep_dispatch_prequantized, prepare_dispatch_prequantized,
                 recv_layout, ep_layout_dispatch, prepare_layout_dispatch, ep_check_quant_e4m3, ep_probe_stream, ep_layout, ep_layout_workspace_bytes, ep_recv_rows, ep_status_string, lib,
                 library_path, prepare_combine, prepare_combine_backward, prepare_dispatch,
                 prepare_dispatch_backward, prepare_layout)

__all__ = ["EP_BF16", "EP_FP8_E4M3", "EP_MXFP8_E4M3", "EP_MXFP4_E2M1", "EpError", "EpShape", "LayoutBuffers", "Prepared", "alloc_recv",
           "ep_abi_version", "prepare_layout", "prepare_dispatch", "prepare_combine",
           "prepare_dispatch_backward", "prepare_combine_backward", "ep_dispatch_backward", "ep_combine_backward",
           "ep_dispatch_prequantized", "prepare_dispatch_prequantized", "ep_check_cvt_e2m1", "recv_layout",
           "ep_layout_dispatch", "prepare_layout_dispatch", "ep_check_quant_e4m3", "ep_probe_stream",
           "ep_check_cvt_bf16", "ep_check_cvt_e4m3", "ep_combine", "ep_dispatch", "ep_layout",
           "ep_layout_workspace_bytes", "ep_recv_rows", "ep_status_string", "lib", "library_path"]
