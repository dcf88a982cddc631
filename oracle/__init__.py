"""CPU oracle of the tiled ViT vision tower -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, calls or falls back to it.

It is a plain, slow, obviously-correct numpy implementation, fp32 end to end,
of the forward pass of the MiniMax-M3 vision tower (MiniMax-M3-Vision README,
"Architecture" table: CLIP-style ViT, 32 layers, hidden 1280, 16 heads, MLP
5120, patch 14, Conv3d patch embed, 3D RoPE, GELU; 2x2 spatial merge with
temporal patch 2; the four-Linear projector).  It shares no code with the HIP
path: the only common module is ``synth`` (seeded random inputs).

Parity status per function is listed in ``oracle.vit``'s docstring.  The
gradients of one block (the backward pass) are in ``oracle.grad``.
"""
from .vit import *  # noqa: F401,F403
from . import grad  # noqa: F401
