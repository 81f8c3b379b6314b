"""MI355X-native int4 lm_head speculative verification.

The compute path is the HIP library built from ``csrc/`` (gfx950 only); the
Python entry points below marshal torch tensors into its C ABI.  Importing
this package loads nothing; the library is loaded on the first call.
"""

__all__ = ["verify", "verify_batch", "verify_batch_noalloc", "verify_mapped", "verify_sampled", "check_weights", "check_vocab_map",
           "workspace_bytes", "load_library",
           "requant_amax", "requant_scales", "requant_pack", "requantize", "context_copy", "stream_read"]


def __getattr__(name):
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
