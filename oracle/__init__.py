"""Plain fp64 CPU oracle of the layer this repository computes on the GPU.

This package is TEST INFRASTRUCTURE.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  The product library (``token_transformer_layer_amd``) never
imports, links or calls anything here, and nothing here imports the product
library: the two share no code.

Every function is pinned by a CPU test against something other than itself
(a pure-Python brute force, finite differences, closed forms, the
tensor-parallel shard-sum identity and the token-slice invariance); the
function docstrings name the passage each one follows.  No function here is
"parity unpinned".
"""
from .layer import *  # noqa: F401,F403
from . import cube, slicing  # noqa: E402,F401
