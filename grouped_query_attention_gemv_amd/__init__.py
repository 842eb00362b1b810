"""MI355X grouped-query attention block (Llama 3.1 8B shapes).

The computation lives in libgqa.so (hand-written gfx950 HIP kernels behind the
C ABI of include/gqa.h); this package is its thin binding.
"""
from .gqa import (  # noqa: F401
    D_MODEL, N_HEADS, N_KV_HEADS, HEAD_DIM, QKV_DIM, ROPE_PAIRS, DECODE_STAGES, PREFILL_STAGES,
    GQAError, HipEvents, block_decode, block_prefill, empty_caches, kcache_by_position, lib,
    rope_table, status_string, vcache_blocks, vcache_read, vcache_write, workspace,
    workspace_bytes, workspace_init, V_BLOCK, SYNC_BYTES, VOCAB_MFMA_MIN_B, DECODE_AUTO,
    DECODE_SPLIT, DECODE_FUSED, OP_PREFILL, OP_DECODE, OP_LAYER_PREFILL, OP_LAYER_DECODE, OP_VOCAB, WS_ERR_WAIT,
    WS_ERR_WO_WAIT, WS_ERR_INIT, WS_ERR_FP16_RANGE, WS_MAGIC, decode_schedule, workspace_errors,
    workspace_off_home, NORM_EPS, layer_decode, layer_prefill, VOCAB, vocab_logits,
    KV_HEAD_COUNTS, wo_to_fp16, block_decode_noalloc, NOALLOC_SCRATCH_BYTES,
)
