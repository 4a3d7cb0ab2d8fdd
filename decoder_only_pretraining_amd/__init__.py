"""MI355X (gfx950) nanochat GPT forward+backward step.

The computation lives in libgptstep.so (HIP kernels behind the C ABI in
include/gpt_step.h); ``binding`` is its ctypes wrapper and ``build``
compiles it in-tree.
"""
from . import binding  # noqa: F401
