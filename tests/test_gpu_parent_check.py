"""The parent-check build (libgdnbeam_check.so, include/gdn_beam_check.h):
decode steps with valid parents give the product library's bits and count
nothing; parent pointers outside [0, W_max) are clamped (no access leaves the
store) and counted once per (request, beam), on the fused scalar-decay,
fused channel-decay and general kernels."""

import ctypes

import numpy as np
import pytest
import torch

from gpu_util import log, run_beam
from linear_attention_beam_gdn_amd import binding as B
from linear_attention_beam_gdn_amd import build, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    lib = ctypes.CDLL(build.CHECK_LIB)
    P, I32 = ctypes.c_void_p, ctypes.c_int32
    lib.gdn_beam_decode_step.argtypes = [ctypes.POINTER(B.GdnShape), ctypes.POINTER(B.GdnStore), I32, I32,
                                         P, P, P, P, P, P, P, P]
    lib.gdn_beam_decode_step.restype = ctypes.c_int
    lib.gdn_debug_bad_parents.argtypes = [P]
    lib.gdn_debug_bad_parents.restype = ctypes.c_int
    return lib


def _decode(L, store, t, W, d, parent, o):
    s = torch.cuda.current_stream().cuda_stream
    rc = L.gdn_beam_decode_step(ctypes.byref(store.shape), ctypes.byref(store.cstore), t, W,
                                parent.data_ptr() if t > 0 else None, d["q"].data_ptr(), d["k"].data_ptr(),
                                d["v"].data_ptr(), d["alpha"].data_ptr(), d["beta"].data_ptr(), o.data_ptr(), s)
    assert rc == B.GDN_OK, rc


@pytest.mark.parametrize("dk,channel", [(128, False), (128, True), (16, False)])
def test_parent_check_build(L, dk, channel):
    R, H, W, T = 2, 2, 20, 3
    inp = synth.make_inputs(R=R, H=H, dk=dk, dv=dk, W=W, L=T, s0_std=0.05, seed=960 + dk, parents="topk",
                            channel_decay=channel)
    _, ref_outs = run_beam(inp, channel)  # the product library
    s = torch.cuda.current_stream().cuda_stream
    assert L.gdn_debug_bad_parents(s) >= 0  # start from zero
    store = B.Store(R, W, H, dk, dk, T, channel_decay=channel, S=torch.from_numpy(inp["S0"]).cuda())
    for t, st in enumerate(inp["steps"]):
        d = B.upload(st)
        o = torch.empty(R, W, H, dk, dtype=torch.float32, device="cuda")
        _decode(L, store, t, W, d, d.get("parent"), o)
        torch.cuda.synchronize()
        assert np.array_equal(o.cpu().numpy(), ref_outs[t]), t
    assert L.gdn_debug_bad_parents(s) == 0
    # step 1 again with four pointers out of range (two requests), each counted once
    d = B.upload(inp["steps"][1])
    bad = d["parent"].clone()
    bad[0, 3], bad[0, 7], bad[1, 0], bad[1, 19] = W + 7, -2, 1 << 20, -1
    o = torch.empty(R, W, H, dk, dtype=torch.float32, device="cuda")
    _decode(L, store, 1, W, d, bad, o)
    assert L.gdn_debug_bad_parents(s) == 4
    assert L.gdn_debug_bad_parents(s) == 0  # reset by the read
    assert torch.isfinite(o).all()
    log(f"[check] d={dk} channel={channel}: bits equal the product library; 4 bad parents counted")
