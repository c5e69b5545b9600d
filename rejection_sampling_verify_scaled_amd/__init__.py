"""MI355X-native speculative-decoding verify step (gfx950 HIP kernels, C ABI).

The entry points mirror include/spec_verify.h:
  spec_verify_greedy(target, offsets, tokens, max_k, ...)
  spec_verify_sample(target, draft, offsets, tokens, temperature, seed, max_k, ...)
They live in ``binding`` and load ``libspecverify.so`` on first use; there is
no CPU fallback.  ``workloads`` holds the seeded synthetic inputs.
"""

__all__ = ["spec_verify_greedy", "spec_verify_sample", "workspace_bytes", "load_library"]


def __getattr__(name):
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
