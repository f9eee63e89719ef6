"""MI355X-native Multi-Token Attention forward (gfx950 HIP kernels behind a C ABI).

Importing the package loads nothing native; the HIP library is loaded on the
first call of ``forward``.
"""
from .inputs import CONFIGS, MTAConfig, generate  # noqa: F401

__all__ = ["CONFIGS", "MTAConfig", "generate", "forward"]


def forward(*args, **kwargs):
    from .binding import forward as _fwd
    return _fwd(*args, **kwargs)
