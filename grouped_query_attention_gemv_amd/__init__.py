"""MI355X grouped-query attention block (Llama 3.1 8B shapes).

The computation lives in libgqa.so (hand-written gfx950 HIP kernels behind the
C ABI of include/gqa.h); this package is its thin binding.
"""
from .gqa import (  # noqa: F401
    D_MODEL, N_HEADS, N_KV_HEADS, HEAD_DIM, QKV_DIM, ROPE_PAIRS, DECODE_STAGES, PREFILL_STAGES,
    GQAError, HipEvents, block_decode, block_prefill, empty_caches, kcache_by_position, lib,
    rope_table, status_string, vcache_blocks, vcache_read, vcache_write, workspace,
    workspace_bytes, V_BLOCK, SYNC_BYTES, DECODE_AUTO, DECODE_SPLIT, DECODE_FUSED,
    decode_schedule, set_decode_schedule, workspace_errors,
    NORM_EPS, layer_decode, layer_prefill, layer_workspace, VOCAB, vocab_logits, KV_HEAD_COUNTS,
)
