"""Device-split all-to-all-v (a2av) for MI355X (gfx950).

W virtual ranks live as W partitions of one GPU's HBM. The exchange, the
offsets, the payload copy and the MoE pack/unpack run in hand-written HIP
kernels behind the C ABI of ``liba2av.so`` (declared in ``include/a2av.h``);
this package is the thin ctypes binding over it. The library is loaded on the
first call and a missing library is an error: there is no fallback path.
"""
from ._binding import *  # noqa: F401,F403
from ._binding import __all__  # noqa: F401
