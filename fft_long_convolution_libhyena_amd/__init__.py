"""libhyena for AMD MI355X: the Hyena operator forward hot path in hand-written HIP.

The compute runs in ``libhyena.so`` (HIP kernels for gfx950 behind the C ABI in
``include/hyena.h``); this package only loads it and marshals torch tensors.
"""
from .binding import (EXPORTS, HyenaError, Plan, Plan2D, Plan3D, LIB_PATH, load_library, kernel_synthesis,  # noqa: F401,E501
                      HYENA_F32, HYENA_BF16, PATH_AUTO, PATH_LDS, PATH_FOURSTEP, PATH_PARTITIONED)

__all__ = ["Plan", "Plan2D", "Plan3D", "HyenaError", "load_library", "kernel_synthesis", "LIB_PATH", "EXPORTS"]
