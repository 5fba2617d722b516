"""MI355X-native Mamba selective scan: a C-ABI HIP library for gfx950.

``binding`` exposes the library's entry points (``ssm_scan_fwd``,
``ssm_state_update``) on torch device tensors; ``inputs`` holds the seeded
synthetic input recipes of the layer shapes the library is measured on.
The shared library itself is loaded on first use, not at import.
"""
from . import binding, inputs  # noqa: F401

__all__ = ["binding", "inputs"]
