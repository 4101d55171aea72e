"""MI355X (gfx950) Blockwise Parallel Transformer layer forward.

The compute lives in libbpt.so (hand-written HIP kernels behind the C ABI in
include/bpt.h); ``binding`` marshals torch tensors into that ABI, and
``layer`` adds small conveniences (tensor upload, workspace allocation).
"""
from .binding import (BPT_BF16, BPT_F32, BptError, BptShape, bpt_debug_attention,  # noqa: F401
                      bpt_debug_intermediates, bpt_layer_algorithmic_flops,
                      bpt_layer_epilogue_rows, bpt_layer_fwd, bpt_layer_fwd_ex,
                      bpt_layer_workspace_bytes, bpt_layer_workspace_bytes_ex,
                      bpt_status_string, bpt_version, make_shape)
