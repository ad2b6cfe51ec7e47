"""Minimal ctypes access to the HIP runtime that PyTorch has loaded: timing
events and stream-capture graphs.  Used by the benchmark and the tests around
the library; the library itself takes a stream and launches on it."""
from __future__ import annotations

import ctypes
from ctypes import POINTER, byref, c_float, c_int, c_size_t, c_uint, c_void_p


def _runtime() -> ctypes.CDLL:
    path = None
    with open("/proc/self/maps") as f:
        for line in f:
            if "libamdhip64" in line:
                path = line.split()[-1]
                break
    return ctypes.CDLL(path or "libamdhip64.so.7")


class HipRuntime:
    # timing-only events: no system-scope fence (cache writeback/invalidate) on record
    EVENT_DISABLE_SYSTEM_FENCE = 0x20000000
    CAPTURE_MODE_THREAD_LOCAL = 1

    def __init__(self):
        h = self.hip = _runtime()
        h.hipEventCreateWithFlags.argtypes = [POINTER(c_void_p), c_uint]
        h.hipEventElapsedTime.argtypes = [POINTER(c_float), c_void_p, c_void_p]
        h.hipEventDestroy.argtypes = [c_void_p]
        h.hipEventRecord.argtypes = [c_void_p, c_void_p]
        h.hipStreamBeginCapture.argtypes = [c_void_p, c_int]
        h.hipStreamEndCapture.argtypes = [c_void_p, POINTER(c_void_p)]
        h.hipGraphInstantiate.argtypes = [POINTER(c_void_p), c_void_p, c_void_p, c_void_p, c_size_t]
        h.hipGraphLaunch.argtypes = [c_void_p, c_void_p]
        h.hipGraphExecDestroy.argtypes = [c_void_p]
        h.hipGraphDestroy.argtypes = [c_void_p]
        self.events = []
        self.graphs = []

    def _ok(self, rc: int, what: str):
        if rc != 0:
            raise RuntimeError(f"{what} failed with HIP error {rc}")

    # -- events ---------------------------------------------------------------
    def event(self) -> int:
        ev = c_void_p()
        self._ok(self.hip.hipEventCreateWithFlags(byref(ev), self.EVENT_DISABLE_SYSTEM_FENCE),
                 "hipEventCreateWithFlags")
        self.events.append(ev.value)
        return ev.value

    def record(self, ev: int, stream: int):
        self._ok(self.hip.hipEventRecord(c_void_p(ev), c_void_p(stream)), "hipEventRecord")

    def ms(self, e0: int, e1: int) -> float:
        out = c_float()
        self._ok(self.hip.hipEventElapsedTime(byref(out), c_void_p(e0), c_void_p(e1)),
                 "hipEventElapsedTime")
        return float(out.value)

    # -- graphs -----------------------------------------------------------------
    def capture(self, stream: int, fn) -> int:
        """Record every launch fn() enqueues on `stream` into an executable graph."""
        self._ok(self.hip.hipStreamBeginCapture(c_void_p(stream), self.CAPTURE_MODE_THREAD_LOCAL),
                 "hipStreamBeginCapture")
        try:
            fn()
        finally:
            graph = c_void_p()
            rc = self.hip.hipStreamEndCapture(c_void_p(stream), byref(graph))
        self._ok(rc, "hipStreamEndCapture")
        exe = c_void_p()
        self._ok(self.hip.hipGraphInstantiate(byref(exe), graph, None, None, 0), "hipGraphInstantiate")
        self.graphs.append((exe.value, graph.value))
        return exe.value

    def launch(self, exe: int, stream: int):
        self._ok(self.hip.hipGraphLaunch(c_void_p(exe), c_void_p(stream)), "hipGraphLaunch")

    def close(self):
        for ev in self.events:
            self.hip.hipEventDestroy(c_void_p(ev))
        for exe, graph in self.graphs:
            self.hip.hipGraphExecDestroy(c_void_p(exe))
            self.hip.hipGraphDestroy(c_void_p(graph))
        self.events, self.graphs = [], []
