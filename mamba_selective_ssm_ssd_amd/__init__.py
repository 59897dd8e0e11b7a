"""Mamba-3 SSM sequence mixer on MI355X (gfx950).

    from mamba_selective_ssm_ssd_amd import prefill, decode_step, State

``capi`` is the ctypes binding of the C ABI (include/m3_ssm.h); ``mixer``
wraps it for torch tensors; ``synth`` draws seeded synthetic inputs.  The
torch-facing names are imported lazily so that ``synth`` works without torch.
"""

_LAZY = ("prefill", "decode_step", "State", "workspace_bytes", "make_shape")


def __getattr__(name):
    if name in _LAZY:
        from . import mixer
        return getattr(mixer, name)
    raise AttributeError(name)
