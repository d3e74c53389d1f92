"""MI355X-native Multi-Token-Prediction draft / verify / rollback path.

The work happens in ``libmtp.so`` (hand-written gfx950 HIP kernels behind the C ABI
of ``include/mtp.h``); ``_lib`` binds that ABI with ctypes and ``head`` wraps it for
PyTorch device tensors and streams.
"""
from ._lib import (CREATE_NO_PACKED_COPY, LIB_PATH, MtpError, mtp_adapt_k, mtp_config,  # noqa: F401
                   mtp_create, mtp_create_ex, mtp_destroy, mtp_draft, mtp_draft_debug,
                   mtp_draft_sample, mtp_get_error, mtp_kv, mtp_kv_catchup, mtp_kv_prefill,
                   mtp_kv_rollback, mtp_refresh_weights, mtp_status_string, mtp_step_weights,
                   mtp_verify, mtp_verify_hidden, mtp_verify_sample, mtp_weights,
                   mtp_workspace_size, mtp_workspace_size_ex)
from .head import MtpCache, MtpHead  # noqa: F401
