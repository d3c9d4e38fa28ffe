"""MI355X (gfx950) hot path of the CSA2 layer of DeepSeek-V4.1-Flash on one GPU.

libcsa2.so (C ABI in include/csa2.h) holds the HIP kernels: MXFP4 encoder,
indexer block scan and pool scan (MFMA), deterministic top-k, and sparse MLA
attention over the MXFP4 main KV plus the FP8 window.  `_lib` is the ctypes
binding (argument marshalling only); `layers` sequences the calls into the
Full / Reindex / Reuse layer modes.
"""
from . import _lib, layers  # noqa: F401
from ._lib import (Csa2Error, encode_entries, index_full, index_pool, quantize_kv, quantize_swa,  # noqa: F401
                   sparse_attn, sparse_attn_rope_bf16, sparse_attn_workspace, topk,
                   topk_workspace)

__all__ = ["Csa2Error", "encode_entries", "index_full", "index_pool", "quantize_kv", "quantize_swa",
           "sparse_attn", "sparse_attn_rope_bf16", "sparse_attn_workspace", "topk",
           "topk_workspace", "layers"]
