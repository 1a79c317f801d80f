"""HIP events with explicit creation flags, for callers of moe_layer.

torch's events cannot be created with HIP's fence flags. A timing event
recorded with a system-scope release makes the GPU write back its L2 at that
point, which idles the device for microseconds between the kernels it
brackets; events created with hipEventDisableSystemFence use a device-scope
release and time the kernels alone. Fork/join events of the second stream
use the same flag plus hipEventDisableTiming.

The HIP runtime used is the one already loaded in the process (torch's), so
the events belong to the same runtime as torch's streams and libmoe.so.
"""
from __future__ import annotations

import ctypes
import re

import torch  # noqa: F401  (loads the HIP runtime first)

HIP_EVENT_DISABLE_TIMING = 0x2
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000

_hip = None


def runtime() -> ctypes.CDLL:
    """The loaded HIP runtime (the copy torch loaded, found in the process map)."""
    global _hip
    if _hip is None:
        path = "libamdhip64.so"
        try:
            with open("/proc/self/maps") as f:
                found = re.findall(r"(/\S*libamdhip64\.so[.\d]*)\s*$", f.read(), flags=re.M)
            if found:
                path = found[0]
        except OSError:
            pass
        h = ctypes.CDLL(path)
        h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        h.hipEventDestroy.argtypes = [ctypes.c_void_p]
        _hip = h
    return _hip


class Event:
    """A hipEvent_t owned by Python (destroyed with the object)."""

    def __init__(self, timing: bool = True):
        torch.cuda.init()
        flags = HIP_EVENT_DISABLE_SYSTEM_FENCE | (0 if timing else HIP_EVENT_DISABLE_TIMING)
        h = ctypes.c_void_p()
        r = runtime().hipEventCreateWithFlags(ctypes.byref(h), flags)
        if r != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({r})")
        self.handle = h.value

    def elapsed_ms(self, end: "Event") -> float:
        """Milliseconds from this event to `end` (both recorded and complete)."""
        ms = ctypes.c_float()
        r = runtime().hipEventElapsedTime(ctypes.byref(ms), self.handle, end.handle)
        if r != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({r})")
        return ms.value

    def __del__(self):
        if getattr(self, "handle", None) and _hip is not None:
            _hip.hipEventDestroy(self.handle)
            self.handle = None
