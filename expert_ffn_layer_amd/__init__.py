"""MI355X-native MoE expert-FFN layer: hand-written HIP kernels for gfx950 behind a C ABI
(``include/moe.h``), with a thin ctypes binding of the same names (``native``)."""
from . import perfmodel  # noqa: F401  (host-side closed forms, no GPU)
