"""MI355X-native CSA / HCA hybrid compressed attention (DeepSeek-V4) hot path.

The compute lives in libcsa.so (HIP kernels for gfx950 behind a C ABI,
include/csa.h); this package is its ctypes binding plus the seeded synthetic
input generator (synth).  Build the library with
`python -m compressed_sparse_long_csa_amd.build`.
"""
from .binding import (BF16, F32, FP8, MXFP4, SPLIT, VARIANT_AUTO, VARIANT_FULL_DIMS,  # noqa: F401
                      VARIANT_HIGH_OCC, VARIANT_LOW_OCC, CsaError, csa_compress, csa_compress_batch, csa_compress_score,
                      csa_compress_score_paged, csa_compress_score_topk, csa_compress_score_topk_paged,
                      csa_select_and_pad,
                      debug_poison_lds,
                      hybrid_attn_decode, hybrid_attn_decode_paged,
                      hybrid_attn_prefill, hybrid_attn_prefill_paged, indexer_score, indexer_score_paged,
                      indexer_score_paged_rows,
                      load_library, row_bytes,
                      topk_noalloc_max_bytes, topk_select, topk_select_noalloc,
                      score_topk_workspace_bytes, topk_workspace_bytes)
