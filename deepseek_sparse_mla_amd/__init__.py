"""MI355X-native DSA sparse-attention path: lightning indexer, top-k, sparse MLA.

The compute lives in libdsa.so (HIP kernels for gfx950 behind a C ABI, see
include/dsa.h); this package is its thin Python binding.  Importing the
package does not load the library; the first call does, and raises if the
library has not been built.
"""
from ._binding import (  # noqa: F401
    DSA_BF16, DSA_F32, DSA_FP8_E4M3FN, DSA_MAX_SHARED_LAYERS, DSA_TOPK_MAX, DsaError, EXPORTS, LIB_PATH,
    Layout, dsa_abi_version, dsa_index_front_end, dsa_index_k_cache_write, dsa_index_q_quant,
    dsa_index_scores, dsa_index_scores_hist, dsa_index_topk, dsa_topk, dsa_topk_after_hist,
    dsa_topk_workspace_size, load_library, mla_workspace, sparse_mla_decode,
    sparse_mla_decode_no_alloc, sparse_mla_decode_shared, dsa_gather_ceiling, dsa_read_ceiling, score_pitch,
    sparse_mla_prefill,
    sparse_mla_workspace_size, topk_workspace,
)
