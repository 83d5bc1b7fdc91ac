"""INT2 rotated-latent MLA decode for AMD MI355X (gfx950).

The compute lives in libmla.so (HIP kernels behind the C ABI in
include/mla.h); this package is its thin Python binding.
"""
from .binding import (  # noqa: F401
    Cache, Dims, GqaCache, GqaDims, MlaError, lib, header_functions, GQA_K_QUERY_COVARIANCE, GQA_K_QUERY_METRIC,
    gqa_append_quant, gqa_calibrate, gqa_decode, gqa_decode_workspace_size, gqa_fit_clip, gqa_prepare_rotation,
    mla_abi_version, mla_append_quant, mla_calibrate_rotation, mla_calibrate_rotation_weighted,
    mla_decode_absorbed, mla_decode_absorbed_noalloc, mla_decode_noalloc_max_workspace, mla_decode_sparse,
    mla_decode_step, mla_index_topk, mla_index_topk_workspace_size,
    mla_decode_workspace_size, mla_fit_clip, mla_fold_absorb_weights, mla_last_error,
    mla_prepare_rotation, mla_set_decode_variant, mla_status_string, mla_timing_enable,
    mla_timing_query, mla_timing_reset,
)
