"""GatedDeltaNet layer for AMD MI355X (gfx950): Python binding of libgdn.so.

Thin ctypes marshalling over the C ABI declared in ``include/gdn.h``: every
step of the layer runs in the library's HIP kernels; PyTorch only provides
device memory and the current stream.  If the library is not built, every
call raises -- there is no fallback.

Pages: "[Qwen3.5 MoE] Add hybrid decoder model" (GatedDeltaNet,
RMSNormGated, depthwise conv1d), "Support Qwen35 SFT" (varlen mode),
"feat(models): dense Qwen3.5 custom attention" (cu_seqlens, one packed row).
"""
from ._binding import (  # noqa: F401
    F32, BF16, GdnError, Shape, lib_path, load,
    max_chunks, chunk_index,
    conv1d, conv1d_bwd, conv1d_bwd_workspace,
    chunk_fwd, chunk_fwd_workspace, chunk_bwd, chunk_bwd_workspace, chunk_fwd_gated, chunk_bwd_gated, chunk_fwd_fp8,
    norm_gate, norm_gate_bwd, norm_gate_bwd_workspace, norm_gate_bwd_noalloc,
    gates, gates_bwd, gates_bwd_workspace,
    recurrent_step, conv1d_step, conv1d_window, conv1d_prefill,
    profile_enable, profile_report, probe_copy, probe_mfma,
)
from .layer import GatedDeltaNetLayer, capture, layer_forward, layer_backward, token_segments  # noqa: F401
