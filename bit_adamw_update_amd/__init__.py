"""Fused 4-bit AdamW optimizer step for MI355X (gfx950).

This package is a thin ctypes binding of the C ABI in ``include/q4adamw.h``
(``libq4adamw.so``): it marshals arguments and nothing else.  Every step of
the optimizer runs in the library's HIP kernels; PyTorch only provides device
memory and the current stream.  Importing works anywhere; loading the
library (first call) raises when it has not been built.
"""
from __future__ import annotations

from .api import (  # noqa: F401
    Q4Config, Q4HParams, Q4Tensor, Q4StateBytes, Q4StateHeader, Q4Error, load_library,
    q4adamw_abi_version, q4adamw_status_string, q4adamw_last_error, q4adamw_default_config,
    q4adamw_validate, q4adamw_workspace_bytes, q4adamw_state_bytes, q4adamw_make_header,
    q4adamw_check_header, q4adamw_host_scalars, q4adamw_codebook, q4adamw_init_state, q4adamw_step,
    q4adamw_dequant_state, q4adamw_flat_offsets, q4adamw_accumulate, q4adamw_grad_stats, q4adamw_grad_norm,
    RECIPE_ZIP_SR, RECIPE_ZE_EDEN, RECIPE_FACTORED, RECIPE_FP32, RECIPE_CUSTOM, RECIPE_BLOCK8,
    CB_NF4, CB_SDYN4, CB_DYN4, CB_DYN4_NZ, CB_LIN4_NZ, CB_SDYN8, CB_DYN8,
    RULE_STATE_RTN, RULE_STATE_SR, RULE_UPDATE_RTN, RULE_UPDATE_SR,
    HP_REUSE_TABLE, HP_CHECK_POINTERS, HP_GRAD_STATS, ACC_FIRST, ACC_LAST, ACC_REUSE_TABLE, TF_LM_HEAD,
)
from .state import Q4State, RECIPE_BY_NAME  # noqa: F401
