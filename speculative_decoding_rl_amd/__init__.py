"""Self-speculative RL rollout step on MI355X (gfx950).

The C library (libsdrl.so, built from csrc/ by build.py) implements the
step: a drafter quantized from the target's own weights proposes gamma tokens
over the shared paged KV cache, the bf16 target verifies gamma+1 positions in
one forward, a lossless rejection sampler decides, the KV tail rolls back, and
a roofline controller toggles speculation and adapts gamma.  This package is
its Python binding (argument marshalling only).
"""
from ._lib import load, lib_path, ErError  # noqa: F401
from .rollout import Engine, History, controller_choose  # noqa: F401
