"""ctypes binding of libcsa_probe.so (include/csa_probe.h): the achievable-peak
probes -- a bf16 matrix-core loop and a streaming read -- timed on torch's
current stream.  Argument marshalling and event timing only."""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcsa_probe.so")
EXPORTS = ("csa_probe_mfma_bf16", "csa_probe_mfma_flops", "csa_probe_read", "csa_probe_lds",
           "csa_probe_lds_bytes")
_lib = None


def lib():
    """The loaded libcsa_probe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                               "`python -m sparse_long_context_pool_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.csa_probe_mfma_bf16.argtypes = [vp, i32, i32, vp]
        L.csa_probe_mfma_bf16.restype = ctypes.c_int
        L.csa_probe_mfma_flops.argtypes = [i32, i32]
        L.csa_probe_mfma_flops.restype = ctypes.c_double
        L.csa_probe_read.argtypes = [vp, sz, vp, i32, vp]
        L.csa_probe_read.restype = ctypes.c_int
        L.csa_probe_lds.argtypes = [vp, i32, i32, i32, vp]
        L.csa_probe_lds.restype = ctypes.c_int
        L.csa_probe_lds_bytes.argtypes = [i32, i32, i32]
        L.csa_probe_lds_bytes.restype = ctypes.c_double
        _lib = L
    return _lib


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _timed(fn, reps):
    """Median milliseconds of `reps` launches, each between its own events."""
    ev = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        ev.append((a, b))
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in ev)
    return t[len(t) // 2]


def mfma_bf16(n_wg: int, iters: int, reps: int = 5):
    """(TFLOP/s, sink) of the matrix-core loop: n_wg workgroups of four waves."""
    sink = torch.empty(n_wg * 256, dtype=torch.float32, device="cuda")

    def run():
        rc = lib().csa_probe_mfma_bf16(ctypes.c_void_p(sink.data_ptr()), n_wg, iters, _stream())
        if rc != 0:
            raise RuntimeError(f"csa_probe_mfma_bf16: hip error {rc}")
    run()
    ms = _timed(run, reps)
    return lib().csa_probe_mfma_flops(n_wg, iters) / (ms * 1e-3) / 1e12, sink


def hbm_read(buf: torch.Tensor, n_wg: int, reps: int = 5):
    """(GB/s, sink) of the streaming read of `buf` (contiguous, 16-byte multiple)."""
    nbytes = buf.numel() * buf.element_size()
    sink = torch.empty(n_wg * 256, dtype=torch.int32, device="cuda")

    def run():
        rc = lib().csa_probe_read(ctypes.c_void_p(buf.data_ptr()), nbytes,
                                  ctypes.c_void_p(sink.data_ptr()), n_wg, _stream())
        if rc != 0:
            raise RuntimeError(f"csa_probe_read: hip error {rc}")
    run()
    ms = _timed(run, reps)
    return nbytes / (ms * 1e-3) / 1e9, sink


def lds_read(mode: int, n_wg: int, iters: int, reps: int = 5):
    """(TB/s over the device, bytes per shader clock per workgroup, sink) of the
    LDS read loop: mode 0 = 16-byte reads, 1 = transposing 8-byte reads.  With
    at most one workgroup per compute unit (n_wg <= CUs) the second figure is
    the compute unit's LDS read rate."""
    sink = torch.empty(2 * n_wg * 512, dtype=torch.int32, device="cuda")

    def run():
        rc = lib().csa_probe_lds(ctypes.c_void_p(sink.data_ptr()), n_wg, iters, mode, _stream())
        if rc != 0:
            raise RuntimeError(f"csa_probe_lds: hip error {rc}")
    run()
    ms = _timed(run, reps)
    total = lib().csa_probe_lds_bytes(n_wg, iters, mode)
    cyc = sink.view(n_wg, 512, 2)[:, 0, 1].cpu().numpy().view("uint32").astype("float64")
    per_cu_clk = total / n_wg / float(cyc.mean())
    return total / (ms * 1e-3) / 1e12, per_cu_clk, sink
