"""MHLA (token-level multi-head linear attention) forward pass for MI355X (gfx950).

The computation lives in libmhla.so (C ABI: include/mhla.h, HIP kernels in
csrc/); :mod:`token_level_head_amd.binding` is a thin ctypes layer over it, and
:mod:`token_level_head_amd.workloads` draws seeded synthetic inputs.  The
binding (and torch) is imported on first use, so the input generator stays
light.
"""
import importlib

_BINDING_NAMES = {
    "LIB_PATH", "MHLA_DTYPE_BF16", "MHLA_DTYPE_F32", "MHLA_ERR_HIP", "MHLA_ERR_INVALID_ARG",
    "MHLA_ERR_NO_MEMORY", "MHLA_ERR_UNSUPPORTED", "MHLA_OK", "MhlaError", "load_library",
    "mhla_block_summaries", "mhla_forward", "mhla_forward_f32", "mhla_forward_path", "MHLA_PATH_STAGED",
    "MHLA_PATH_FUSED", "mhla_last_error", "mhla_mix_summaries",
    "mhla_output", "mhla_status_string", "mhla_summary_floats", "mhla_unpack_summaries", "mhla_version",
    "mhla_workspace_bytes", "mhla_decode_state_bytes", "mhla_decode_step",
    "mhla_backward_workspace_bytes", "mhla_backward", "mhla_forward_ex", "MHLA_OPT_CAUSAL",
    "MHLA_OPT_NO_NORMALIZER", "MHLA_OPT_OUT_BF16", "MHLA_OPT_W_PER_HEAD", "mhla_forward_blocks",
    "mhla_release_workspace", "mhla_debug_fail_workspace", "mhla_forward_noalloc", "MHLA_NOALLOC_SCRATCH_BYTES",
    "mhla_backward_ex", "mhla_decode_step_ex", "MHLA_PATH_PAIR",
}


def __getattr__(name):
    if name in _BINDING_NAMES:
        return getattr(importlib.import_module(".binding", __name__), name)
    raise AttributeError(name)


def __dir__():
    return sorted(_BINDING_NAMES | set(globals()))
