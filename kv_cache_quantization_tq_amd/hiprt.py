"""HIP runtime helpers for timing and graph capture (measurement
infrastructure; the codec itself is the C ABI in libtq.so).

HipEvent   a timing event created with hipEventDisableSystemFence:
           recording it performs no system-scope cache write-back and
           invalidation, which would otherwise add several microseconds to
           every marked step and slow the kernel that follows.
HipGraph   launches recorded by a callable, captured with the runtime's
           stream capture on a stream of their own (default priority,
           non-blocking), instantiated once and launched as one submission.
           The callable runs with that stream as torch's current stream, so
           the binding's calls launch into it.

Calls go to the HIP runtime already loaded in the process (the one the
codec library and torch use).
"""
from __future__ import annotations

import ctypes
import gc

_P = ctypes.c_void_p
_hip = None

HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000
HIP_STREAM_NON_BLOCKING = 0x1
HIP_STREAM_CAPTURE_MODE_GLOBAL = 0


def hip():
    """The loaded HIP runtime, with the argument types of the calls used here."""
    global _hip
    if _hip is None:
        path = None
        with open("/proc/self/maps") as f:
            for ln in f:
                if "libamdhip64" in ln:
                    path = ln.split()[-1]
                    break
        if path is None:
            raise RuntimeError("the HIP runtime is not loaded in this process")
        L = ctypes.CDLL(path)
        L.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(_P), ctypes.c_uint]
        L.hipEventRecord.argtypes = [_P, _P]
        L.hipEventSynchronize.argtypes = [_P]
        L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), _P, _P]
        L.hipEventDestroy.argtypes = [_P]
        L.hipStreamCreateWithFlags.argtypes = [ctypes.POINTER(_P), ctypes.c_uint]
        L.hipStreamSynchronize.argtypes = [_P]
        L.hipStreamDestroy.argtypes = [_P]
        L.hipStreamBeginCapture.argtypes = [_P, ctypes.c_int]
        L.hipStreamEndCapture.argtypes = [_P, ctypes.POINTER(_P)]
        L.hipGraphInstantiate.argtypes = [ctypes.POINTER(_P), _P, _P, ctypes.c_char_p, ctypes.c_size_t]
        L.hipGraphLaunch.argtypes = [_P, _P]
        L.hipGraphExecDestroy.argtypes = [_P]
        L.hipGraphDestroy.argtypes = [_P]
        _hip = L
    return _hip


def _check(status, what):
    if status != 0:
        raise RuntimeError(f"{what} failed (hipError {status})")


class HipEvent:
    def __init__(self, stream):
        self.stream = stream
        self.ev = _P()
        _check(hip().hipEventCreateWithFlags(ctypes.byref(self.ev), HIP_EVENT_DISABLE_SYSTEM_FENCE),
               "hipEventCreateWithFlags")

    def record(self):
        _check(hip().hipEventRecord(self.ev, self.stream), "hipEventRecord")

    def elapsed_time(self, end):
        """Milliseconds from this event to `end` (both complete)."""
        ms = ctypes.c_float()
        _check(hip().hipEventSynchronize(end.ev), "hipEventSynchronize")
        _check(hip().hipEventElapsedTime(ctypes.byref(ms), self.ev, end.ev), "hipEventElapsedTime")
        return ms.value

    def __del__(self):
        if _hip is not None and self.ev:
            _hip.hipEventDestroy(self.ev)


class HipGraph:
    def __init__(self, torch, record):
        L = hip()
        s = _P()
        _check(L.hipStreamCreateWithFlags(ctypes.byref(s), HIP_STREAM_NON_BLOCKING), "hipStreamCreateWithFlags")
        self.stream = s.value
        self.graph, self.exec = _P(), _P()
        torch.cuda.synchronize()
        # No garbage collection while capturing: a collected object's
        # destructor may call the HIP runtime (free memory, destroy an event
        # or a graph), which a global-mode capture forbids and the runtime
        # answers by aborting the process.
        gc.collect()
        gc_was_on = gc.isenabled()
        gc.disable()
        try:
            _check(L.hipStreamBeginCapture(self.stream, HIP_STREAM_CAPTURE_MODE_GLOBAL), "hipStreamBeginCapture")
            try:
                with torch.cuda.stream(torch.cuda.ExternalStream(self.stream)):
                    record()
            except BaseException:
                # end the capture, drop what it recorded, and report the caller's error
                L.hipStreamEndCapture(self.stream, ctypes.byref(self.graph))
                self.close()
                raise
            _check(L.hipStreamEndCapture(self.stream, ctypes.byref(self.graph)), "hipStreamEndCapture")
        finally:
            if gc_was_on:
                gc.enable()
        _check(L.hipGraphInstantiate(ctypes.byref(self.exec), self.graph, None, None, 0), "hipGraphInstantiate")

    def launch(self):
        _check(hip().hipGraphLaunch(self.exec, self.stream), "hipGraphLaunch")

    def synchronize(self):
        _check(hip().hipStreamSynchronize(self.stream), "hipStreamSynchronize")

    def close(self):
        L = hip()
        if self.stream:
            L.hipStreamSynchronize(self.stream)
        if self.exec:
            L.hipGraphExecDestroy(self.exec)
            self.exec = _P()
        if self.graph:
            L.hipGraphDestroy(self.graph)
            self.graph = _P()
        if self.stream:
            L.hipStreamDestroy(self.stream)
            self.stream = None
