"""Fused QK-RMSNorm + 3D M-RoPE joint text+image attention for MI355X (gfx950).

The compute runs in the HIP library ``libmrope_attn.so`` (built from
``csrc/``) behind a C ABI; ``mrope_attn`` below marshals torch tensors into
that ABI. ``workloads`` draws the seeded synthetic inputs.
"""

from . import workloads  # noqa: F401


def __getattr__(name):
    # the binding loads the shared library on first use and fails loudly
    # when it is missing; importing the package alone never needs it
    if name in ("mrope_attn", "MraError", "lib", "workspace_size", "validate", "KPRO_AUTO",
                "KPRO_FUSED", "KPRO_PREPASS"):
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
