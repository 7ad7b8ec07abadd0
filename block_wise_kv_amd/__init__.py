"""block_wise_kv_amd: the Fast-dLLM block-decoding hot path on MI355X.

The compute runs in libfdllm.so (HIP kernels for gfx950, C ABI declared in
include/fdllm.h); this package holds the ctypes binding and the build step.
"""
from .fdllm import (  # noqa: F401
    BF16, F32, MODE, UNMASK_ADVANCE_BLOCK, FdllmError, SeqDesc, AttnDesc,
    attn_desc, block_attn, block_attn_workspace, kv_refresh, kv_refresh_layers, lib, lmhead_pack, lmhead_packed_bytes,
    lmhead_unmask_threshold, lmhead_unmask_topk, lmhead_unmask_workspace, new_workspace, seq_desc,
    set_debug, set_lmhead_tuning, set_timing_events, set_tuning, unmask_threshold, unmask_threshold_static,
    unmask_topk, unmask_workspace, version,
    workspace_init,
)
