"""Streaming rates of this GPU at fixed read:write mixes, from the hand-written
reference kernel in k_stream.hip (measurement only; not part of the decode
path).

A mix (rd, wr) moves rd bytes read for every wr bytes written, with fully
coalesced 16-byte accesses over buffers far larger than the 256 MB Infinity
Cache.  For each mix the launch shape (workgroups) and store kind (plain or
non-temporal) are swept, and the best rate is kept: the fastest this kernel
streams that mix on this GPU.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgdnmeasure.so")

# (reads, writes) built into the reference kernel, by read fraction
MIXES = [(0, 1), (1, 2), (2, 3), (4, 5), (1, 1), (5, 4), (3, 2), (2, 1), (1, 0)]
UNIT = 4096  # bytes per block

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build the package first")
        L = ctypes.CDLL(LIB_PATH)
        L.gdn_stream_run.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_longlong, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        L.gdn_stream_run.restype = ctypes.c_int
        L.gdn_stream_run_timed.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_longlong, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_void_p]
        L.gdn_stream_run_timed.restype = ctypes.c_int
        L.gdn_timing_event_create.argtypes = []
        L.gdn_timing_event_create.restype = ctypes.c_void_p
        L.gdn_timing_event_destroy.argtypes = [ctypes.c_void_p]
        L.gdn_timing_event_destroy.restype = None
        L.gdn_timing_elapsed_us.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        L.gdn_timing_elapsed_us.restype = ctypes.c_double
        _lib = L
    return _lib


def mix_rate(torch, stream, rd, wr, total_bytes=2 << 30, wgs=(1024, 2048, 4096, 8192), reps=10):
    """Best rate (GB/s, read + written bytes over time) of the mix (rd, wr),
    with the launch shape and store kind that gave it."""
    units = total_bytes // ((rd + wr) * UNIT) // 4 * 4
    src = torch.empty(max(1, units * rd * UNIT // 4), dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty(max(1024, units * wr * UNIT // 4), dtype=torch.float32, device="cuda")
    nbytes = units * (rd + wr) * UNIT
    best = (0.0, None)
    h = ctypes.c_void_p(stream.cuda_stream)
    for n_wg in wgs:
        for nts in (0, 1):
            if wr == 0 and nts:
                continue

            def go():
                rc = lib().gdn_stream_run(rd, wr, src.data_ptr(), dst.data_ptr(), units, n_wg, nts, h)
                if rc != 0:
                    raise RuntimeError(f"gdn_stream_run({rd}, {wr}) returned {rc}")

            go()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a.record(stream)
            for _ in range(reps):
                go()
            b.record(stream)
            torch.cuda.synchronize()
            gbs = nbytes / (a.elapsed_time(b) / reps * 1e-3) / 1e9
            if gbs > best[0]:
                best = (gbs, {"workgroups": n_wg, "nontemporal_stores": bool(nts)})
    del src, dst
    return {"GBps": best[0], **best[1], "read_fraction": rd / (rd + wr), "bytes": nbytes}


def all_rates(torch, stream, **kw):
    """Best rate of every built mix, keyed 'r<rd>w<wr>'."""
    return {f"r{rd}w{wr}": mix_rate(torch, stream, rd, wr, **kw) for rd, wr in MIXES}


def rate_at(rates, read_fraction):
    """The measured rate (GB/s) at a read fraction, piecewise linear between
    the measured mixes."""
    pts = sorted((v["read_fraction"], v["GBps"]) for v in rates.values())
    xs = [p[0] for p in pts]
    ys = [p[1] for p in pts]
    if read_fraction <= xs[0]:
        return ys[0]
    for i in range(1, len(xs)):
        if read_fraction <= xs[i]:
            f = (read_fraction - xs[i - 1]) / (xs[i] - xs[i - 1])
            return ys[i - 1] + f * (ys[i] - ys[i - 1])
    return ys[-1]


class ReadFlush:
    """Evicts the 256 MB Infinity Cache by reading a 1 GiB buffer with the
    reads-only mix: the cache then holds clean lines of that buffer and none
    of the next kernel's data, and no dirty line of the flush is left to be
    written back while the next kernel runs (a copy would leave up to the
    cache's size of them)."""

    def __init__(self, torch, nbytes=1 << 30):
        self.units = nbytes // UNIT // 4 * 4
        self.src = torch.zeros(self.units * UNIT // 4, dtype=torch.float32, device="cuda")
        self.dst = torch.empty(1024, dtype=torch.float32, device="cuda")

    def __call__(self, stream):
        rc = lib().gdn_stream_run(1, 0, self.src.data_ptr(), self.dst.data_ptr(), self.units, 1024, 0,
                                  ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"gdn_stream_run(1, 0) returned {rc}")



class KernelEvents:
    """HIP event pairs for kernel-bracketing timing: handed to a launch
    (gdn_beam_decode_step_timed, gdn_stream_run_timed), the runtime records
    the first as the kernel starts and the second as it completes, so their
    difference is the kernel's execution alone, with no event command in the
    stream and no system-scope fence (see gdn_timing_event_create)."""

    def __init__(self, n):
        self.pairs = []
        for _ in range(n):
            a, b = lib().gdn_timing_event_create(), lib().gdn_timing_event_create()
            if not a or not b:
                self.close()
                raise RuntimeError("gdn_timing_event_create failed")
            self.pairs.append((a, b))

    def elapsed_us(self):
        """Microseconds of every pair, in order (waits for each)."""
        out = []
        for a, b in self.pairs:
            us = lib().gdn_timing_elapsed_us(a, b)
            if us < 0:
                raise RuntimeError("gdn_timing_elapsed_us failed (an event pair was not recorded)")
            out.append(us)
        return out

    def close(self):
        for a, b in self.pairs:
            lib().gdn_timing_event_destroy(a)
            lib().gdn_timing_event_destroy(b)
        self.pairs = []


def empty_kernel_us(torch, stream, reps=20, workgroups=256):
    """Median kernel time, as the runtime brackets it (KernelEvents), of a
    launch that does almost nothing (256 workgroups reading 16 KiB), each
    after the read-only sweep: what any kernel launched this way costs."""
    flush = ReadFlush(torch)
    src = torch.zeros(4 * UNIT // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty(1024, dtype=torch.float32, device="cuda")
    h = ctypes.c_void_p(stream.cuda_stream)
    ev = KernelEvents(reps)
    try:
        for a, b in ev.pairs:
            flush(stream)
            rc = lib().gdn_stream_run_timed(1, 0, src.data_ptr(), dst.data_ptr(), 4, workgroups, 0, h, a, b)
            if rc != 0:
                raise RuntimeError(f"gdn_stream_run_timed(1, 0) returned {rc}")
        times = ev.elapsed_us()
    finally:
        ev.close()
    del flush
    return sorted(times)[len(times) // 2]


def empty_launch_us(torch, stream, reps=20, workgroups=256):
    """Median time between HIP events recorded around a launch that does
    almost nothing (256 workgroups reading 16 KiB), each after the read-only
    sweep: the floor that a launch timed with its own event pair pays."""
    flush = ReadFlush(torch)
    src = torch.zeros(4 * UNIT // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty(1024, dtype=torch.float32, device="cuda")
    h = ctypes.c_void_p(stream.cuda_stream)
    times = []
    for _ in range(reps):
        flush(stream)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        rc = lib().gdn_stream_run(1, 0, src.data_ptr(), dst.data_ptr(), 4, workgroups, 0, h)
        b.record(stream)
        torch.cuda.synchronize()
        if rc != 0:
            raise RuntimeError(f"gdn_stream_run(1, 0) returned {rc}")
        times.append(a.elapsed_time(b) * 1e3)
    del flush
    return sorted(times)[len(times) // 2]


def main():
    """Prints the best rate of every mix as a markdown table, and what a
    near-empty launch costs, timed both ways."""
    import torch

    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    rates = all_rates(torch, stream)
    print("| mix (read:write) | read fraction | best GB/s | of 8 TB/s | workgroups | non-temporal stores |")
    print("|---|---|---|---|---|---|")
    for key, v in rates.items():
        rd, wr = key[1:].split("w")
        print(f"| {rd}:{wr} | {v['read_fraction']:.3f} | {v['GBps']:.0f} | {v['GBps'] / 8000:.3f} | "
              f"{v['workgroups']} | {'yes' if v['nontemporal_stores'] else 'no'} |", flush=True)
    print(f"\nA launch of 256 workgroups reading 16 KiB, after the read-only sweep: {empty_kernel_us(torch, stream):.1f} us "
          f"as the runtime brackets the kernel, {empty_launch_us(torch, stream):.1f} us between HIP events recorded "
          f"around it (medians of 20).", flush=True)


if __name__ == "__main__":
    main()
