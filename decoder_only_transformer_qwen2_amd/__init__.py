"""Qwen2 decoder forward (prefill + KV-cached greedy decode) on AMD MI355X.

The compute lives in libqw.so (HIP kernels for gfx950 behind the C ABI of
include/qw.h); this package is its ctypes binding.
"""
from .qw import (  # noqa: F401
    EXPORTED, LIB_PATH, QW_KV_BLOCK, Model, QwError, device_tensors, load_library, make_config, qw_check_ids,
    qw_check_numerics, qw_config, qw_create, qw_create_paged, qw_decode_step, qw_decode_step_noalloc, qw_destroy,
    qw_generate, qw_get_finished, qw_get_positions, qw_get_state, qw_kernel_names, qw_kv_blocks, qw_last_error,
    qw_layer_weights, qw_peak_copy, qw_peak_mfma, qw_prefill, qw_prefill_ragged, qw_set_eos, qw_set_graph,
    qw_set_sampling, qw_timing_enable, qw_timing_read, qw_weights,
)
