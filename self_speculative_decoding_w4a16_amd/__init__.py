"""Self-speculative decoding with a 4-bit (W4A16) substitute draft on one
AMD Instinct MI355X (gfx950).  The hot path lives in libsubspec.so (HIP
kernels behind the C ABI of include/subspec.h); this package holds the
ctypes binding, the device-model container and the cycle driver."""
from . import _lib  # noqa: F401
from ._lib import SubspecError, lib  # noqa: F401
