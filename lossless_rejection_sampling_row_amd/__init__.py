"""MI355X-native speculative-decoding verify sampler (lossless, mu-gated rejection sampling).

The work is done by the HIP library ``libsv_verify.so``, behind the C-ABI in
``include/sv_verify.h``. ``verify_batch`` marshals torch tensors into that
ABI. Names are resolved lazily, so importing the package (for example to use
``workloads``) loads neither torch nor the library.
"""
_BINDING_NAMES = {
    "ABI_VERSION", "SvError", "library_path", "load_library", "verify_batch", "workspace_bytes",
    "verify_sampler_match", "verify_batch_static", "filter_thresholds", "row_acceptance", "expand_schedule", "split_row_diag", "set_tuning", "get_tuning",
}


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
