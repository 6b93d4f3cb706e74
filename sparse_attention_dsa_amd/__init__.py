"""DeepSeek Sparse Attention (DSA) step for AMD MI355X (gfx950).

Lightning-indexer scores, top-K selection and sparse MQA-mode MLA over a
paged latent / indexer-key cache, as hand-written HIP kernels behind the C ABI
in ``include/dsa.h``.  ``binding`` is the thin Python front end.
"""
from .binding import (Batch, DsaError, check_batch, decode_step, decode_step_fused, decode_step_timed,  # noqa: F401
                      indexer_scores, lib, sparse_mla_decode, sparse_mla_decode_layers, sparse_mla_prefill, topk,
                      workspace_size)
