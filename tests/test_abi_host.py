"""The C ABI on the host: the library loads, exports what the header
declares, and rejects bad arguments before touching the GPU (CPU only)."""

import ctypes
import subprocess

import pytest

from linear_attention_beam_gdn_amd import binding as B

FAKE = 0x10000  # aligned, never dereferenced: validation fails first


@pytest.fixture(scope="module")
def L():
    return B.lib()


def shape(**kw):
    d = dict(R=2, W_max=8, H=2, dk=128, dv=128, L_max=4, decay_kind=0, H_k=0)
    d.update(kw)
    return B.GdnShape(**d)


def store(**kw):
    d = dict(S=FAKE, rec_delta=FAKE, rec_k=FAKE, rec_alpha=FAKE, anc=FAKE)
    d.update(kw)
    return B.GdnStore(**d)


def decode(L, sh=None, st=None, t=1, W_t=4, parent=FAKE, q=FAKE, k=FAKE, v=FAKE, alpha=FAKE,
           beta=FAKE, o=FAKE, timed=False):
    sh = shape() if sh is None else sh
    st = store() if st is None else st
    args = (ctypes.byref(sh), ctypes.byref(st), t, W_t, parent, q, k, v, alpha, beta, o, None)
    if timed:  # event handles that are never used: validation fails first
        return L.gdn_beam_decode_step_timed(*args, FAKE, FAKE)
    return L.gdn_beam_decode_step(*args)


def test_exports_every_header_function(L):
    names = B.header_functions()
    assert set(names) == {"gdn_beam_decode_step", "gdn_decode_merge_step", "gdn_materialize",
                          "gdn_log_merge", "gdn_status_string", "gdn_abi_version",
                          "gdn_split_workspace_bytes", "gdn_decode_step_split",
                          "gdn_decode_step_split_noalloc", "gdn_beam_decode_step_timed"}
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    for n in names:
        assert n in exported, n
        assert hasattr(L, n)


def test_version_and_status_strings(L):
    assert L.gdn_abi_version() == 7
    for s in (B.GDN_OK, B.GDN_EINVAL, B.GDN_EUNSUPPORTED, B.GDN_EHIP, B.GDN_ESCRATCH, 12345):
        assert isinstance(B.status_string(s), str) and B.status_string(s)


@pytest.mark.parametrize("timed", [False, True], ids=["untimed", "timed"])
def test_decode_validation(L, timed):
    """gdn_beam_decode_step and gdn_beam_decode_step_timed reject the same
    arguments with the same codes."""
    E, U = B.GDN_EINVAL, B.GDN_EUNSUPPORTED
    P = ctypes.POINTER
    fn = L.gdn_beam_decode_step_timed if timed else L.gdn_beam_decode_step
    ev = (FAKE, FAKE) if timed else ()
    assert fn(P(B.GdnShape)(), ctypes.byref(store()), 0, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, *ev) == E
    assert fn(ctypes.byref(shape()), P(B.GdnStore)(), 0, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, *ev) == E

    def dec(L, **kw):
        return decode(L, timed=timed, **kw)

    assert dec(L, sh=shape(R=0)) == E
    assert dec(L, sh=shape(H=0)) == E
    assert dec(L, sh=shape(L_max=0)) == E
    assert dec(L, sh=shape(L_max=B.GDN_MAX_STEPS + 1)) == E
    assert dec(L, sh=shape(dk=96, dv=96)) == U
    assert dec(L, sh=shape(dk=128, dv=64)) == U
    assert dec(L, sh=shape(dk=256, dv=64)) == U
    assert dec(L, sh=shape(dk=512, dv=512)) == U
    assert dec(L, sh=shape(dk=256, dv=128, decay_kind=1)) == U  # channel decay: d_k = 128 only
    assert dec(L, sh=shape(dk=128, dv=256, decay_kind=2, W_max=1)) == U  # plain: square only
    assert dec(L, sh=shape(decay_kind=2)) == U  # the plain (RWKV6) rule: sequences only
    assert dec(L, sh=shape(decay_kind=3)) == U
    assert dec(L, sh=shape(H=4, H_k=3)) == E  # key heads must divide the value heads
    assert dec(L, sh=shape(H_k=-1)) == E
    assert dec(L, t=-1) == E
    assert dec(L, t=4) == E
    assert dec(L, W_t=0) == E
    assert dec(L, W_t=9) == E
    assert dec(L, t=1, parent=None) == E
    assert dec(L, t=1, parent=FAKE + 2) == E
    for name in ("q", "k", "v", "alpha", "beta", "o"):
        assert dec(L, **{name: None}) == E, name
        assert dec(L, **{name: FAKE + 8}) == E, name
    for name in ("S", "rec_delta", "rec_k", "rec_alpha", "anc"):
        assert dec(L, st=store(**{name: None})) == E, name
        assert dec(L, st=store(**{name: FAKE + 4})) == E, name


def test_materialize_and_merge_validation(L):
    E = B.GDN_EINVAL
    sh, st = shape(), store()
    m = lambda t=1, rb=FAKE, n=3, out=FAKE: L.gdn_materialize(ctypes.byref(sh), ctypes.byref(st), t,
                                                              rb, n, out, None)
    assert m(n=0) == B.GDN_OK  # nothing to do, nothing enqueued
    assert m(n=-1) == E
    assert m(t=4) == E
    assert m(t=-1) == E
    assert m(rb=None) == E
    assert m(out=FAKE + 4) == E
    g = lambda n_rec=2, beam=0: L.gdn_log_merge(ctypes.byref(sh), ctypes.byref(st), n_rec, beam, None)
    assert g(n_rec=0) == E
    assert g(n_rec=5) == E
    assert g(beam=-1) == E
    assert g(beam=8) == E
    for bad in (shape(dk=48, dv=48), shape(dk=256, dv=256, decay_kind=1)):
        assert L.gdn_log_merge(ctypes.byref(bad), ctypes.byref(st), 1, 0, None) == B.GDN_EUNSUPPORTED


def test_binding_refuses_host_tensors():
    import torch
    st = B.Store.__new__(B.Store)
    st.R, st.H, st.Hk, st.dk, st.dv, st.channel_decay = 1, 1, 1, 16, 16, False
    st.device = torch.device("cuda", 0)
    x = torch.zeros(1, 1, 1, 16, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device tensor"):
        B.decode_step(st, 0, 1, None, x, x, x, torch.zeros(1, 1, 1), torch.zeros(1, 1, 1))


def test_decode_merge_validation(L):
    E, U = B.GDN_EINVAL, B.GDN_EUNSUPPORTED
    seq = shape(W_max=1)

    def dm(sh=seq, st=None, t=3, q=FAKE, k=FAKE, v=FAKE, alpha=FAKE, beta=FAKE, o=FAKE):
        st = store() if st is None else st
        return L.gdn_decode_merge_step(ctypes.byref(sh), ctypes.byref(st), t, q, k, v, alpha, beta, o, None)

    assert dm(sh=shape(W_max=8)) == U  # beams: merge with gdn_log_merge instead
    assert dm(sh=shape(W_max=1, dk=96, dv=96)) == U
    assert dm(sh=shape(W_max=1, dk=128, dv=256)) == U  # the sequence kernel: square shapes
    assert dm(t=-1) == E
    assert dm(t=4) == E
    for name in ("q", "k", "v", "alpha", "beta", "o"):
        assert dm(**{name: None}) == E, name
        assert dm(**{name: FAKE + 8}) == E, name
    for name in ("S", "rec_delta", "rec_k", "rec_alpha", "anc"):
        assert dm(st=store(**{name: None})) == E, name


def split(L, sh=None, st=None, t=1, n_split=2, shared=1, merge=0, ws=FAKE, ws_bytes=1 << 30):
    sh = shape(W_max=1) if sh is None else sh
    st = store() if st is None else st
    return L.gdn_decode_step_split(ctypes.byref(sh), ctypes.byref(st), t, n_split, shared, merge, FAKE, FAKE,
                                   FAKE, FAKE, FAKE, FAKE, ws, ws_bytes, None)


def test_split_workspace_size(L):
    # one replay preparation per (sequence, head): 2 d_k probes, 2 x 16 dot products, k_t . q_t, padding
    sh = shape(R=128, W_max=1, H=32)
    assert L.gdn_split_workspace_bytes(ctypes.byref(sh)) == 128 * 32 * (2 * 128 + 2 * 16 + 4) * 4
    assert L.gdn_split_workspace_bytes(ctypes.byref(shape(R=0))) == 0


def test_split_validation(L):
    E, U = B.GDN_EINVAL, B.GDN_EUNSUPPORTED
    need = L.gdn_split_workspace_bytes(ctypes.byref(shape(W_max=1)))
    assert split(L, sh=shape(W_max=4)) == U                    # beams: sequences only
    assert split(L, sh=shape(W_max=1, dk=64, dv=64)) == U      # d = 128 only
    assert split(L, n_split=3) == U and split(L, n_split=8) == U
    assert split(L, t=4) == E and split(L, t=-1) == E
    assert split(L, merge=2) == E and split(L, shared=2) == E
    assert split(L, ws=None) == E                             # the shared arm needs a workspace
    assert split(L, ws=FAKE + 4) == E                         # misaligned
    assert split(L, ws_bytes=need - 1) == E                   # too small
    assert split(L, st=store(rec_k=FAKE + 2)) == E
    assert split(L, sh=shape(W_max=1, decay_kind=7)) == U


def test_noalloc_split_rejects_before_touching_the_gpu(L):
    """The no-alloc entry point refuses a shape whose preparation would not fit
    its built-in scratch buffer (and the split path's own errors) before any
    HIP call."""
    def call(sh, shared=1, n_split=2, st=None):
        st = store() if st is None else st
        return L.gdn_decode_step_split_noalloc(ctypes.byref(sh), ctypes.byref(st), 0, n_split, shared, 0, FAKE,
                                               FAKE, FAKE, FAKE, FAKE, FAKE, None)
    per = (2 * 128 + 2 * 16 + 4) * 4
    too_many = B.GDN_SPLIT_SCRATCH_BYTES // per + 1
    assert call(shape(R=too_many, W_max=1, H=1)) == B.GDN_ESCRATCH
    assert call(shape(R=too_many, W_max=1, H=1), shared=0, n_split=3) == B.GDN_EUNSUPPORTED
    assert call(shape(W_max=4), shared=0) == B.GDN_EUNSUPPORTED
    assert call(shape(R=0, W_max=1)) == B.GDN_EINVAL
    assert call(shape(W_max=1), shared=0, st=store(S=FAKE + 8)) == B.GDN_EINVAL



def test_parent_check_library_exports():
    """libgdnbeam_check.so exports everything gdn_beam.h declares plus the
    counter reader gdn_beam_check.h declares."""
    import os
    import re

    from linear_attention_beam_gdn_amd import build

    out = subprocess.run(["nm", "-D", "--defined-only", build.CHECK_LIB], capture_output=True, text=True,
                         check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    hdr = open(os.path.join(os.path.dirname(B.HEADER), "gdn_beam_check.h")).read()
    hdr = re.sub(r"/\*.*?\*/", "", hdr, flags=re.S)
    extra = re.findall(r"^\s*\w+\s+(gdn_\w+)\s*\(", hdr, flags=re.M)
    assert extra == ["gdn_debug_bad_parents"]
    for n in B.header_functions() + extra:
        assert n in exported, n
    prod = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True,
                          check=True).stdout
    assert "gdn_debug_bad_parents" not in prod  # the product build has no counter


def test_stamps_library_exports():
    """libgdnbeam_stamps.so exports everything gdn_beam.h declares plus the
    clock-stamp readers of the two fused kernels; the product library has
    none of them."""
    from linear_attention_beam_gdn_amd import build

    def exported(path):
        out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True, check=True).stdout
        return {ln.split()[-1] for ln in out.splitlines() if ln.strip()}

    st = exported(build.STAMPS_LIB)
    readers = ["gdn_stamps_read", "gdn_kda_stamps_read", "gdn_stamps_clock_khz"]
    for n in B.header_functions() + readers:
        assert n in st, n
    prod = exported(B.LIB_PATH)
    for n in readers:
        assert n not in prod, n
