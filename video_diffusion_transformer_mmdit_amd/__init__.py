"""MI355X-native dual-stream MMDiT block core.

Thin Python binding over the C ABI of ``libmmdit.so`` (header ``include/mmdit.h``): each
function marshals torch tensors (device memory, current stream) into the C call of the
same name.  Every step of the computation runs in the library's HIP kernels; there is no
Python or PyTorch compute fallback, and importing a missing library raises.
"""
from ._abi import (  # noqa: F401
    ATTN8_SPLIT_BYTES, ATTN_SPLIT_BYTES, Attn8Operands, BF16, F16, F32, FP8_E4M3, STAGES, STAGE_COUNT, EPI_GATED_RES, EPI_GELU, EPI_NONE, MmditError, Rope3D, BlockDims,
    WS_G, WS_H, WS_MOD, WS_QKV, WS_SPLIT, WS_W1, WS_W2, WS_WO, WS_WQKV, WS_X1,
    WS_XQ, WS_XS, WS_Q8, WS_QS, WS_K8, WS_KS, WS_V8T, WS_VS, WS_COUNT, SCALE_KEYS, fp8_block_weights,
    abi_version, attn8_quantize, block_fwd, cast, block_workspace_bytes, block_workspace_offsets, joint_attention, joint_attention_8bit,
    joint_attention_noalloc, NOALLOC_SCRATCH_BYTES, MATRIX_KEYS,
    lib, library_path, linear, linear_fp8, lite_merge, lite_unpatchify, modulate_ln, modulation, qk_norm_rope, quantize_fp8, timestep_embed,
)
