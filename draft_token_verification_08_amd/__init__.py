"""libspecverify: the batched verify-and-sample step of speculative decoding and
the MTP token shift/insert, as hand-written HIP kernels for MI355X (gfx950).

The C ABI is declared in include/specverify.h; this package is its Python
binding (torch tensors in, device pointers and the current stream out).
"""
from ._lib import (  # noqa: F401
    SV_BF16, SV_EALIGN, SV_EHIP, SV_EINVAL, SV_EWORKSPACE, SV_F32, SV_FLAG_BAD_TEMP,
    SV_FLAG_BAD_PARENT, SV_FLAG_BAD_UNIFORM, SV_FLAG_LEN_CLAMPED, SV_FLAG_ROW_CLAMPED, SV_FLAG_TOKEN_OOR, SV_FLAG_TREE_TRUNCATED,
    SV_FLAG_ZERO_RESIDUAL,
    SV_MAX_DRAFT,
    SV_OK, Prepared, SpecVerifyError, Workspace, lib, mtp_shift_insert, prepare_mtp_shift_insert,
    prepare_spec_verify_greedy, prepare_spec_verify_greedy_mtp, prepare_spec_verify_sample,
    prepare_spec_verify_greedy_lmhead, prepare_spec_verify_sample_ex, prepare_spec_verify_sample_mtp,
    prepare_sv_sample_rows, prepare_spec_verify_tree_greedy, prepare_spec_verify_tree_sample, spec_verify_tree_sample, sv_tree_rounds,
    spec_verify_greedy, spec_verify_greedy_lmhead, spec_verify_tree_greedy, spec_verify_greedy_mtp, spec_verify_sample, sv_lmhead_logits_debug,
    spec_verify_sample_ex, spec_verify_sample_ex_noalloc, spec_verify_sample_mtp, sv_sample_rows, draft_row_stats, sv_residual_weights_debug, sv_softmax_rows_debug, sv_workspace_bytes, sv_workspace_clear,
)
