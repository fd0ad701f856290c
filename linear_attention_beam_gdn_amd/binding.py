"""ctypes binding of libgdnbeam.so (C ABI in include/gdn_beam.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  PyTorch provides device memory and the stream; there is no CPU
fallback, and a missing library raises.
"""

from __future__ import annotations

import ctypes
import os
import re

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libgdnbeam.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "gdn_beam.h")

GDN_OK, GDN_EINVAL, GDN_EUNSUPPORTED, GDN_EHIP, GDN_ESCRATCH = 0, -1, -2, -3, -4
GDN_SPLIT_SCRATCH_BYTES = 8 << 20
GDN_DECAY_SCALAR, GDN_DECAY_CHANNEL, GDN_DECAY_CHANNEL_PLAIN = 0, 1, 2
GDN_MAX_STEPS = 16


class GdnShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("R", "W_max", "H", "dk", "dv", "L_max", "decay_kind", "H_k")]


class GdnStore(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("S", "rec_delta", "rec_k", "rec_alpha", "anc")]


class GdnError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} (status {status})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libgdnbeam.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m linear_attention_beam_gdn_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I32 = ctypes.c_void_p, ctypes.c_int32
        L.gdn_beam_decode_step.argtypes = [ctypes.POINTER(GdnShape), ctypes.POINTER(GdnStore), I32, I32,
                                           P, P, P, P, P, P, P, P]
        L.gdn_beam_decode_step.restype = ctypes.c_int
        L.gdn_beam_decode_step_timed.argtypes = [ctypes.POINTER(GdnShape), ctypes.POINTER(GdnStore), I32, I32,
                                                 P, P, P, P, P, P, P, P, P, P]
        L.gdn_beam_decode_step_timed.restype = ctypes.c_int
        L.gdn_materialize.argtypes = [ctypes.POINTER(GdnShape), ctypes.POINTER(GdnStore), I32, P, I32, P, P]
        L.gdn_materialize.restype = ctypes.c_int
        L.gdn_log_merge.argtypes = [ctypes.POINTER(GdnShape), ctypes.POINTER(GdnStore), I32, I32, P]
        L.gdn_log_merge.restype = ctypes.c_int
        L.gdn_decode_merge_step.argtypes = [ctypes.POINTER(GdnShape), ctypes.POINTER(GdnStore), I32,
                                            P, P, P, P, P, P, P]
        L.gdn_decode_merge_step.restype = ctypes.c_int
        L.gdn_split_workspace_bytes.argtypes = [ctypes.POINTER(GdnShape)]
        L.gdn_split_workspace_bytes.restype = ctypes.c_size_t
        L.gdn_decode_step_split.argtypes = [ctypes.POINTER(GdnShape), ctypes.POINTER(GdnStore), I32, I32, I32,
                                            I32, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.gdn_decode_step_split.restype = ctypes.c_int
        L.gdn_decode_step_split_noalloc.argtypes = [ctypes.POINTER(GdnShape), ctypes.POINTER(GdnStore), I32, I32,
                                                    I32, I32, P, P, P, P, P, P, P]
        L.gdn_decode_step_split_noalloc.restype = ctypes.c_int
        L.gdn_status_string.argtypes = [ctypes.c_int]
        L.gdn_status_string.restype = ctypes.c_char_p
        L.gdn_abi_version.argtypes = []
        L.gdn_abi_version.restype = ctypes.c_int
        _lib = L
    return _lib


def header_functions() -> list[str]:
    """Names of the functions include/gdn_beam.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(gdn_\w+)\s*\(", text, flags=re.M)


def status_string(status: int) -> str:
    return lib().gdn_status_string(int(status)).decode()


def _ptr(x) -> int | None:
    return None if x is None else x.data_ptr()


def _stream(stream, device) -> int | None:
    """The given stream, else the current stream of the store's device."""
    s = torch.cuda.current_stream(device) if stream is None else stream
    if s.device != device:
        raise ValueError(f"stream is on {s.device}, the store on {device}")
    return s.cuda_stream


def _check(t: torch.Tensor, name: str, dtypes, shape, device=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor (there is no CPU path)")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the store on {device}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")


_BF16 = (torch.bfloat16, torch.int16)


class Store:
    """Caller-owned record / ancestry store (device memory from PyTorch).

    S [R,H,dk,dv] FP32, rec_delta [L,R,W,H,dv] FP32 (bf16 with the plain
    update rule, whose update vectors are v itself), rec_k [L,R,W,Hk,dk] bf16,
    rec_alpha [L,R,W,H,A] FP32, anc [L,R,W,L] int32.
    """

    def __init__(self, R, W_max, H, dk, dv, L_max, channel_decay=False, device="cuda", S=None,
                 plain_update=False, Hk=None):
        self.R, self.W_max, self.H, self.dk, self.dv, self.L_max = R, W_max, H, dk, dv, L_max
        self.Hk = H if Hk is None else Hk
        if self.Hk < 1 or H % self.Hk:
            raise ValueError("Hk (key heads) must divide H")
        if plain_update and not channel_decay:
            raise ValueError("the plain (RWKV6) update rule comes with per-channel decay")
        self.channel_decay = bool(channel_decay)
        self.plain_update = bool(plain_update)
        self.A = dk if channel_decay else 1
        if S is not None:
            _check(S, "S", (torch.float32,), (R, H, dk, dv))
            device = S.device  # the records live beside the given state
        f32 = dict(dtype=torch.float32, device=device)
        self.S = torch.zeros(R, H, dk, dv, **f32) if S is None else S
        self.device = self.S.device
        self.rec_delta = torch.zeros(L_max, R, W_max, H, dv, dtype=torch.bfloat16 if plain_update else torch.float32,
                                     device=device)
        self.rec_k = torch.zeros(L_max, R, W_max, self.Hk, dk, dtype=torch.bfloat16, device=device)
        self.rec_alpha = torch.zeros(L_max, R, W_max, H, self.A, **f32)
        self.anc = torch.zeros(L_max, R, W_max, L_max, dtype=torch.int32, device=device)
        kind = GDN_DECAY_CHANNEL_PLAIN if plain_update else (GDN_DECAY_CHANNEL if channel_decay else GDN_DECAY_SCALAR)
        self.shape = GdnShape(R, W_max, H, dk, dv, L_max, kind, self.Hk)
        self.cstore = GdnStore(_ptr(self.S), _ptr(self.rec_delta), _ptr(self.rec_k),
                               _ptr(self.rec_alpha), _ptr(self.anc))


def decode_step(store: Store, t, W_t, parent, q, k, v, alpha, beta, o=None, stream=None, events=None):
    """One decode step (gdn_beam_decode_step); returns o [R,W_t,H,dv] FP32.
    ``events``: a pair of HIP event handles (ints) that the runtime records as
    the step's kernel starts and completes (gdn_beam_decode_step_timed)."""
    R, H, dk, dv, dev = store.R, store.H, store.dk, store.dv, store.device
    _check(q, "q", _BF16, (R, W_t, store.Hk, dk), dev)
    _check(k, "k", _BF16, (R, W_t, store.Hk, dk), dev)
    _check(v, "v", _BF16, (R, W_t, H, dv), dev)
    a_shape = (R, W_t, H, dk) if store.channel_decay else (R, W_t, H)
    _check(alpha, "alpha", (torch.float32,), a_shape, dev)
    _check(beta, "beta", (torch.float32,), (R, W_t, H), dev)
    if t > 0:
        _check(parent, "parent", (torch.int32,), (R, W_t), dev)
    if o is None:
        o = torch.empty(R, W_t, H, dv, dtype=torch.float32, device=dev)
    _check(o, "o", (torch.float32,), (R, W_t, H, dv), dev)
    args = (ctypes.byref(store.shape), ctypes.byref(store.cstore), t, W_t, _ptr(parent) if t > 0 else None,
            _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(o), _stream(stream, store.device))
    if events is None:
        rc = lib().gdn_beam_decode_step(*args)
    else:
        rc = lib().gdn_beam_decode_step_timed(*args, events[0], events[1])
    if rc != GDN_OK:
        raise GdnError(rc, "gdn_beam_decode_step_timed" if events is not None else "gdn_beam_decode_step")
    return o


def materialize(store: Store, t, rb, out=None, stream=None):
    """Dense states after step t of the (request, beam) pairs rb [n,2] int32."""
    n = int(rb.shape[0])
    _check(rb, "rb", (torch.int32,), (n, 2), store.device)
    if out is None:
        out = torch.empty(n, store.H, store.dk, store.dv, dtype=torch.float32, device=store.device)
    _check(out, "S_out", (torch.float32,), (n, store.H, store.dk, store.dv), store.device)
    rc = lib().gdn_materialize(ctypes.byref(store.shape), ctypes.byref(store.cstore), t, _ptr(rb), n,
                               _ptr(out), _stream(stream, store.device))
    if rc != GDN_OK:
        raise GdnError(rc, "gdn_materialize")
    return out


def decode_merge_step(store: Store, t, q, k, v, alpha, beta, o=None, stream=None):
    """Decode token t of independent sequences and fold the full log into the
    base in the same pass (gdn_decode_merge_step); returns o [R,1,H,dv] FP32."""
    R, H, dk, dv, dev = store.R, store.H, store.dk, store.dv, store.device
    _check(q, "q", _BF16, (R, 1, store.Hk, dk), dev)
    _check(k, "k", _BF16, (R, 1, store.Hk, dk), dev)
    _check(v, "v", _BF16, (R, 1, H, dv), dev)
    _check(alpha, "alpha", (torch.float32,), (R, 1, H, dk) if store.channel_decay else (R, 1, H), dev)
    _check(beta, "beta", (torch.float32,), (R, 1, H), dev)
    if o is None:
        o = torch.empty(R, 1, H, dv, dtype=torch.float32, device=dev)
    _check(o, "o", (torch.float32,), (R, 1, H, dv), dev)
    rc = lib().gdn_decode_merge_step(ctypes.byref(store.shape), ctypes.byref(store.cstore), t, _ptr(q), _ptr(k),
                                     _ptr(v), _ptr(alpha), _ptr(beta), _ptr(o), _stream(stream, store.device))
    if rc != GDN_OK:
        raise GdnError(rc, "gdn_decode_merge_step")
    return o


def split_workspace_bytes(store: Store) -> int:
    """Bytes of the workspace the shared-preparation arm of
    decode_step_split needs for this store (gdn_split_workspace_bytes)."""
    return int(lib().gdn_split_workspace_bytes(ctypes.byref(store.shape)))


def decode_step_split(store: Store, t, n_split, shared_prep, merge, q, k, v, alpha, beta, o=None,
                      workspace=None, stream=None):
    """Token t of independent sequences with d_v cut into n_split value tiles
    (gdn_decode_step_split); shared_prep forms the replay preparation once in
    ``workspace`` (a device tensor of at least split_workspace_bytes bytes),
    else every tile forms it; merge folds the full log as decode_merge_step
    does.  Returns o [R,1,H,dv] FP32."""
    R, H, dk, dv, dev = store.R, store.H, store.dk, store.dv, store.device
    _check(q, "q", _BF16, (R, 1, store.Hk, dk), dev)
    _check(k, "k", _BF16, (R, 1, store.Hk, dk), dev)
    _check(v, "v", _BF16, (R, 1, H, dv), dev)
    _check(alpha, "alpha", (torch.float32,), (R, 1, H, dk) if store.channel_decay else (R, 1, H), dev)
    _check(beta, "beta", (torch.float32,), (R, 1, H), dev)
    if o is None:
        o = torch.empty(R, 1, H, dv, dtype=torch.float32, device=dev)
    _check(o, "o", (torch.float32,), (R, 1, H, dv), dev)
    ws, ws_bytes = None, 0
    if workspace is not None:
        if not workspace.is_cuda or workspace.device != dev or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous device tensor on the store's device")
        ws, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    rc = lib().gdn_decode_step_split(ctypes.byref(store.shape), ctypes.byref(store.cstore), t, n_split,
                                     int(bool(shared_prep)), int(bool(merge)), _ptr(q), _ptr(k), _ptr(v),
                                     _ptr(alpha), _ptr(beta), _ptr(o), ws, ws_bytes, _stream(stream, store.device))
    if rc != GDN_OK:
        raise GdnError(rc, "gdn_decode_step_split")
    return o


def decode_step_split_noalloc(store: Store, t, n_split, shared_prep, merge, q, k, v, alpha, beta, o,
                              stream=None):
    """decode_step_split with the library's built-in scratch buffer instead of
    a workspace (gdn_decode_step_split_noalloc): nothing is allocated, so the
    output ``o`` [R,1,H,dv] FP32 must be given."""
    R, H, dk, dv, dev = store.R, store.H, store.dk, store.dv, store.device
    _check(q, "q", _BF16, (R, 1, store.Hk, dk), dev)
    _check(k, "k", _BF16, (R, 1, store.Hk, dk), dev)
    _check(v, "v", _BF16, (R, 1, H, dv), dev)
    _check(alpha, "alpha", (torch.float32,), (R, 1, H, dk) if store.channel_decay else (R, 1, H), dev)
    _check(beta, "beta", (torch.float32,), (R, 1, H), dev)
    _check(o, "o", (torch.float32,), (R, 1, H, dv), dev)
    rc = lib().gdn_decode_step_split_noalloc(ctypes.byref(store.shape), ctypes.byref(store.cstore), t, n_split,
                                             int(bool(shared_prep)), int(bool(merge)), _ptr(q), _ptr(k), _ptr(v),
                                             _ptr(alpha), _ptr(beta), _ptr(o), _stream(stream, store.device))
    if rc != GDN_OK:
        raise GdnError(rc, "gdn_decode_step_split_noalloc")
    return o


def log_merge(store: Store, n_rec, beam=0, stream=None):
    """Fold the first n_rec records of `beam`'s chain into store.S in place."""
    rc = lib().gdn_log_merge(ctypes.byref(store.shape), ctypes.byref(store.cstore), n_rec, beam,
                             _stream(stream, store.device))
    if rc != GDN_OK:
        raise GdnError(rc, "gdn_log_merge")


def upload(arrays: dict, device="cuda") -> dict:
    """Copy a dict of numpy input arrays to device tensors of the ABI's dtypes
    (uint16 bf16 bit patterns -> torch.bfloat16, float32, int32)."""
    import numpy as np

    out = {}
    for name, a in arrays.items():
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            out[name] = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
        elif a.dtype in (np.float32, np.int32):
            out[name] = torch.from_numpy(a).to(device)
        else:
            raise TypeError(f"{name}: unexpected dtype {a.dtype}")
    return out
