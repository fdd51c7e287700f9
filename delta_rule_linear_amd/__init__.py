"""KLA (Kaczmarz Linear Attention) prefill and decode on MI355X (gfx950).

The compute runs in libkla.so (hand-written HIP kernels behind a C ABI,
include/kla.h).  This package is its Python binding:

    from delta_rule_linear_amd import kla_fwd_chunked, kla_decode_step

The binding is loaded on first use; if libkla.so has not been built
(``python -m delta_rule_linear_amd.build``) that first use raises.
"""
__all__ = ["kla_fwd_chunked", "kla_decode_step", "kla_fwd_chunked_ex", "kla_decode_step_ex",
           "kla_fwd_chunked_split", "kla_fwd_chunked_split_noalloc", "kla_fwd_chunked_kda",
           "kla_decode_step_kda",
           "kla_fwd_chunked_ccq", "kla_decode_step_ccq", "kla_ccq_state_floats",
           "kla_fwd_chunked_workspace_size", "kla_bwd_chunked", "kla_bwd_chunked_workspace_size",
           "kla_fwd_chunked_split_workspace_size", "kla_status_string", "kla_version", "KLAError",
           "lib_path"]


def __getattr__(name):
    if name in __all__:
        from . import kla as _kla
        return getattr(_kla, name)
    raise AttributeError(name)
