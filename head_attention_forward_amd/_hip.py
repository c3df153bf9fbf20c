"""Minimal ctypes access to HIP events (the runtime torch already loaded).

Used to hand raw hipEvent_t handles to the *_timed entry points of libmha
and to read elapsed times; import torch before calling (it loads the
runtime, and the same shared object is reused here)."""

import ctypes

import torch  # noqa: F401  (loads the HIP runtime)

_rt = None


def runtime():
    global _rt
    if _rt is None:
        rt = ctypes.CDLL("libamdhip64.so.7")
        rt.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        rt.hipEventCreateWithFlags.restype = ctypes.c_int
        rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
        rt.hipEventDestroy.restype = ctypes.c_int
        rt.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        rt.hipEventSynchronize.restype = ctypes.c_int
        rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                           ctypes.c_void_p]
        rt.hipEventElapsedTime.restype = ctypes.c_int
        _rt = rt
    return _rt


class EventPool:
    """n raw HIP events (default flags, timing enabled) as a ctypes array."""

    def __init__(self, n):
        rt = runtime()
        self.n = n
        self.array = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            st = rt.hipEventCreateWithFlags(ctypes.byref(h), 0)
            if st != 0:
                raise RuntimeError(f"hipEventCreateWithFlags failed ({st})")
            self.array[i] = h.value

    def ptr(self, offset=0):
        """Pointer to events[offset:]."""
        return ctypes.cast(ctypes.byref(self.array, offset * ctypes.sizeof(ctypes.c_void_p)),
                           ctypes.c_void_p)

    def elapsed_ms(self, i, j):
        rt = runtime()
        st = rt.hipEventSynchronize(self.array[j])
        if st != 0:
            raise RuntimeError(f"hipEventSynchronize failed ({st})")
        out = ctypes.c_float()
        st = rt.hipEventElapsedTime(ctypes.byref(out), self.array[i], self.array[j])
        if st != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({st})")
        return float(out.value)

    def close(self):
        rt = runtime()
        for i in range(self.n):
            if self.array[i]:
                rt.hipEventDestroy(self.array[i])
                self.array[i] = None
