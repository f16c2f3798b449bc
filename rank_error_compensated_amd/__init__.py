"""SERQ's quantized linear layer on AMD Instinct MI355X (gfx950).

The compute lives in ``_lib/libserq.so`` (HIP kernels behind the C ABI in
``include/serq.h``); :mod:`rank_error_compensated_amd.binding` is its ctypes
binding.  Importing this package loads nothing; the library is loaded, and a
missing build reported, on the first call into it.
"""
from .binding import (PreparedLayer, SerqError, lib, serq_act_bytes, serq_flatten_act,  # noqa: F401
                      serq_layout, serq_linear, serq_linear_q, serq_linear_workspace_bytes,
                      serq_prepare_weights, serq_quant_act, serq_query_layout, serq_rmsnorm_quant,
                      serq_swiglu_quant, serq_weight_error, serq_l2qer_sizes, serq_l2qer_prepare,
                      serq_l2qer_workspace_bytes, serq_l2qer_intermediate, serq_l2qer_linear_q,
                      serq_l2qer_linear)
