"""Launch markers (se_set_launch_events) on the GPU (MI355X), through the C ABI.

Armed events are taken two per kernel launch, in launch order, and the dispatch stamps
them with the kernel's start and end.  Checked on the one-read step (four launches at
this shape: sweep, contraction, range merge, scaled reduction): the count of events used, that every start precedes its end and the next
kernel's start, that the durations add up to no more than the bracketed call, that a
list too short for every launch leaves the later launches unmarked, that disarming
stops the marking, and that the outputs are bit for bit those of an unmarked call.
"""
import ctypes
import sys

import numpy as np
import pytest
import torch

from diffusion_self_conditioning_amd import workloads as wl

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from diffusion_self_conditioning_amd import _binding as B
    from diffusion_self_conditioning_amd import api

DEV = "cuda:0"
DISABLE_SYSTEM_FENCE = 0x20000000


def say(*a):
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


class Events:
    """Raw HIP events of the runtime this process already runs (the one the library uses)."""

    def __init__(self):
        torch.cuda.init()
        path = next(ln.split()[-1] for ln in open("/proc/self/maps") if "libamdhip64" in ln)
        self.hip = ctypes.CDLL(path)
        self.live = []

    def create(self, n):
        out = []
        for _ in range(n):
            h = ctypes.c_void_p()
            assert self.hip.hipEventCreateWithFlags(ctypes.byref(h),
                                                    ctypes.c_uint(DISABLE_SYSTEM_FENCE)) == 0
            out.append(h.value)
        self.live += out
        return out

    def record(self, ev):
        stream = torch.cuda.current_stream().cuda_stream
        assert self.hip.hipEventRecord(ctypes.c_void_p(ev), ctypes.c_void_p(stream)) == 0

    def ms(self, a, b):
        t = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(t), ctypes.c_void_p(a),
                                            ctypes.c_void_p(b)) == 0
        return t.value

    def close(self):
        for h in self.live:
            self.hip.hipEventDestroy(ctypes.c_void_p(h))
        self.live = []


def test_markers_time_each_launch_and_change_nothing():
    L, V, s, e, d = 256, 30000, 0, 30000, 512
    rng = np.random.default_rng(61)
    x = (rng.standard_normal((L, V)) * 3).astype(np.float32)
    tab = wl.fp32_to_bf16_bits((rng.standard_normal((e - s, d)) * 0.02).astype(np.float32))
    x_t, w_t = torch.from_numpy(x).to(DEV), torch.from_numpy(tab).to(DEV)
    ws = api.step_onepass_workspace(L, V, s, e, d, DEV)
    f = dict(device=DEV, dtype=torch.float32)

    def outputs():
        return (torch.empty((L, d), **f), torch.empty(L, **f), torch.empty(L, **f),
                torch.empty(L, **f), torch.empty(L, device=DEV, dtype=torch.int32))

    def call(o):
        B.se_soft_embed_step_onepass(x_t, s, e, w_t, 1.5, *o, ws)

    ref = outputs()
    call(ref)
    torch.cuda.synchronize()
    ev = Events()
    try:
        # enough events for every launch
        marks, bracket = ev.create(16), ev.create(2)
        got = outputs()
        say("markers: armed with 16 events")
        ev.record(bracket[0])
        B.se_set_launch_events(marks)
        call(got)
        used = B.se_launch_events_used()
        B.se_set_launch_events([])
        ev.record(bracket[1])
        torch.cuda.synchronize()
        assert used % 2 == 0 and used >= 4, used
        n = used // 2
        dur = [ev.ms(marks[2 * j], marks[2 * j + 1]) for j in range(n)]
        gaps = [ev.ms(marks[2 * j - 1], marks[2 * j]) for j in range(1, n)]
        total = ev.ms(bracket[0], bracket[1])
        say("launches", n, "durations ms", dur, "gaps ms", gaps, "call ms", total)
        assert all(t > 0 for t in dur)
        assert all(g >= 0 for g in gaps)
        assert ev.ms(bracket[0], marks[0]) >= 0 and ev.ms(marks[used - 1], bracket[1]) >= 0
        assert sum(dur) + sum(gaps) <= total * 1.0001
        for a, b in zip(ref, got):
            assert torch.equal(a, b)
        # a list with room for one launch: only the first is marked
        short = ev.create(3)
        B.se_set_launch_events(short)
        call(got)
        assert B.se_launch_events_used() == 2
        B.se_set_launch_events([])
        torch.cuda.synchronize()
        assert ev.ms(short[0], short[1]) > 0
        # disarmed: nothing is taken
        call(got)
        assert B.se_launch_events_used() == 0
        torch.cuda.synchronize()
        for a, b in zip(ref, got):
            assert torch.equal(a, b)
    finally:
        B.se_set_launch_events([])
        torch.cuda.synchronize()
        ev.close()
