"""CPU oracle (test infrastructure only; never imported by the product path)."""
from .ref import (  # noqa: F401
    attend, compress, csa_query, e4m3_decode, hca_query, kv_fp8_decode, mxfp4_decode, mxfp4_quantize,
    indexer_scores, rms_norm, rope_rotate, sparse_rows, topk_select, visible, window_rows,
)
