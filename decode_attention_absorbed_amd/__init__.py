"""MI355X-native absorbed-MLA sparse decode attention (DeepSeek-V3.2-Exp).

The compute path is libmla_decode.so (hand-written HIP for gfx950, C ABI in
include/mla_decode.h); ``mla`` is its ctypes binding.
"""
from . import mla  # noqa: F401
