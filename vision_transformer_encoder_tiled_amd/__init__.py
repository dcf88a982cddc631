"""Tiled ViT vision tower for AMD MI355X (gfx950).

The compute path is the HIP library ``libvt.so`` (C ABI in ``include/vt.h``);
this package is its Python binding.  Importing it raises if the library has
not been built (``python -m vision_transformer_encoder_tiled_amd.build``):
there is no CPU fallback.
"""
from ._lib import *  # noqa: F401,F403
from ._lib import LIB, LIB_PATH, EXPORTED, VtError, TowerWeights  # noqa: F401
