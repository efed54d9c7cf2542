"""MI355X-native chunked forward of Kimi Delta Attention (KDA).

The compute path is the HIP library ``libkda.so`` (C ABI in ``include/kda.h``);
``kda`` is its ctypes binding.  Build with ``python -m gated_delta_rule_chunked_amd.build``.
"""
from .kda import (  # noqa: F401
    KDA_CHUNK, KDA_FLAG_BETA_LOGITS, KDA_FLAG_CKPT_BF16, KDA_FLAG_STATE_BF16, KdaBwdDhuArgs, KdaError, KdaFwdArgs,
    alloc_workspace, kda_bwd_dhu, kda_bwd_dhu_raw, kda_bwd_dhu_workspace_bytes, kda_debug_unpack, kda_fwd,
    kda_fwd_inter, kda_fwd_intra, kda_fwd_no_alloc_raw, kda_fwd_raw, kda_fwd_scan_plan, kda_fwd_workspace_bytes, kda_strerror, load_library,
    make_args, make_bwd_args, max_chunks, num_chunks,
)
