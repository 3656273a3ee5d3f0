"""Thin Python binding of libstreamkl.so (the C ABI in include/streamkl.h).

Argument marshalling only: torch supplies device memory (outputs and the
split-K workspace) and the current HIP stream; every step of the
computation runs in the library's HIP kernels.  There is no fallback: if the
library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libstreamkl.so")

OK, ERR_INVALID, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = range(5)
F32, BF16 = 0, 1
BWD_AUTO, BWD_FUSED, BWD_SEPARATE, BWD_DK_ONLY, BWD_DQ_ONLY = 0, 1, 2, 3, 4


class StreamKLError(RuntimeError):
    def __init__(self, status: int, what: str, hip_error: int = 0):
        self.status = status
        self.hip_error = hip_error
        msg = f"{what}: {_lib().streamkl_status_string(status).decode()} (status {status})"
        if status == ERR_HIP:
            msg += f", hipError {hip_error}"
        super().__init__(msg)


class Shape(ctypes.Structure):
    # kv_heads1/kv_heads2: key heads of each model (0 = H, one per query head);
    # q_len/k_len: host arrays of B lengths for ragged batches (NULL = full)
    _fields_ = [("B", ctypes.c_int64), ("H", ctypes.c_int64), ("n_q", ctypes.c_int64), ("n_k", ctypes.c_int64),
                ("d1", ctypes.c_int32), ("d2", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("kv_heads1", ctypes.c_int32), ("kv_heads2", ctypes.c_int32),
                ("q_len", ctypes.POINTER(ctypes.c_int64)), ("k_len", ctypes.POINTER(ctypes.c_int64)),
                ("q_off", ctypes.POINTER(ctypes.c_int64)), ("k_off", ctypes.POINTER(ctypes.c_int64))]

    def set_lengths(self, q_len=None, k_len=None):
        """Ragged batch: per batch element query and key lengths (sequences of
        B ints, or None for the padded sizes).  The arrays live on this object."""
        for name, v in (("q_len", q_len), ("k_len", k_len)):
            if v is None:
                setattr(self, name, None)
                continue
            v = [int(x) for x in v]
            if len(v) != self.B:
                raise ValueError(f"{name} needs {self.B} lengths")
            arr = (ctypes.c_int64 * len(v))(*v)
            setattr(self, "_" + name, arr)  # keep the array alive
            setattr(self, name, ctypes.cast(arr, ctypes.POINTER(ctypes.c_int64)))
        return self

    def set_offsets(self, q_off, k_off):
        """Packed batch: B + 1 query and key row offsets (sequences one after
        another in every head).  The arrays live on this object."""
        for name, v in (("q_off", q_off), ("k_off", k_off)):
            v = [int(x) for x in v]
            if len(v) != self.B + 1:
                raise ValueError(f"{name} needs {self.B + 1} offsets")
            arr = (ctypes.c_int64 * len(v))(*v)
            setattr(self, "_" + name, arr)
            setattr(self, name, ctypes.cast(arr, ctypes.POINTER(ctypes.c_int64)))
        return self


ABI_VERSION = 5
INVALID_BYTES = (1 << 64) - 1  # STREAMKL_INVALID_BYTES


class Launch(ctypes.Structure):
    _fields_ = [("num_splits", ctypes.c_int32), ("bwd_mode", ctypes.c_int32),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t)]


_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m attention_kl_divergence_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        sp, lp = ctypes.POINTER(Shape), ctypes.POINTER(Launch)
        lib.streamkl_fwd.argtypes = [vp, vp, vp, vp, i32, f32, f32, vp, vp, vp, sp, lp, vp]
        lib.streamkl_fwd.restype = i32
        lib.streamkl_bwd.argtypes = [i32, vp, vp, vp, vp, i32, f32, f32, vp, vp, vp, vp, vp, vp, sp, lp, vp]
        lib.streamkl_bwd.restype = i32
        lib.streamkl_bwd_joint.argtypes = [vp, vp, vp, vp, i32, f32, f32, vp, vp, vp, vp, vp, vp, vp, vp, sp, lp, vp]
        lib.streamkl_bwd_joint.restype = i32
        lib.streamkl_kl_loss.argtypes = [vp, vp, ctypes.c_int64, vp, vp]
        lib.streamkl_kl_loss.restype = i32
        lib.streamkl_fwd_loss.argtypes = [vp, vp, vp, vp, i32, f32, f32, vp, vp, vp, vp, vp, sp, lp, vp]
        lib.streamkl_fwd_loss.restype = i32
        lib.streamkl_fwd_workspace_bytes.argtypes = [sp, i32, lp]
        lib.streamkl_fwd_workspace_bytes.restype = sz
        lib.streamkl_fwd_loss_workspace_bytes.argtypes = [sp, i32, lp]
        lib.streamkl_fwd_loss_workspace_bytes.restype = sz
        lib.streamkl_bwd_workspace_bytes.argtypes = [sp, i32, i32, lp]
        lib.streamkl_bwd_workspace_bytes.restype = sz
        lib.streamkl_fwd_plan.argtypes = [sp, i32, lp]
        lib.streamkl_fwd_plan.restype = i32
        lib.streamkl_bwd_plan.argtypes = [sp, i32, i32, lp]
        lib.streamkl_bwd_plan.restype = i32
        lib.streamkl_status_string.argtypes = [i32]
        lib.streamkl_status_string.restype = ctypes.c_char_p
        lib.streamkl_last_hip_error.argtypes = []
        lib.streamkl_last_hip_error.restype = i32
        lib.streamkl_version.argtypes = []
        lib.streamkl_version.restype = i32
        if lib.streamkl_version() != ABI_VERSION:
            raise RuntimeError(f"{LIB_PATH} has ABI version {lib.streamkl_version()}, this binding needs "
                               f"{ABI_VERSION}: rebuild it")
        _LIB = lib
    return _LIB


def library():
    """The loaded ctypes library (raises if it is not built)."""
    return _lib()


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return F32
    if t == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t}; expected float32 or bfloat16")


def make_shape(B, H, n_q, n_k, d1, d2, dtype, kv_heads1=0, kv_heads2=0) -> Shape:
    code = dtype if isinstance(dtype, int) else _dtype_code(dtype)
    return Shape(B, H, n_q, n_k, d1, d2, code, kv_heads1, kv_heads2)


def shape_of(q1, k1, q2, k2) -> Shape:
    for t in (q1, k1, q2, k2):
        if t.dim() != 4:
            raise ValueError("Q and K tensors must be [B, H, N, d]")
        if not t.is_contiguous():
            raise ValueError("Q and K tensors must be contiguous")
        if t.dtype != q1.dtype:
            raise ValueError("Q1, K1, Q2, K2 must share one dtype")
        if t.device != q1.device:
            raise ValueError("Q1, K1, Q2, K2 must be on one device")
    B, H, n_q, d1 = q1.shape
    n_k = k1.shape[2]
    d2 = q2.shape[3]
    # K_t may have fewer heads than Q_t (grouped key heads): [B, kv_heads_t, n_k, d_t]
    kv1, kv2 = k1.shape[1], k2.shape[1]
    if (tuple(k1.shape) != (B, kv1, n_k, d1) or tuple(q2.shape) != (B, H, n_q, d2)
            or tuple(k2.shape) != (B, kv2, n_k, d2) or H % kv1 or H % kv2):
        raise ValueError("inconsistent Q/K shapes")
    return make_shape(B, H, n_q, n_k, d1, d2, q1.dtype, 0 if kv1 == H else kv1, 0 if kv2 == H else kv2)


def packed_shape_of(q1, k1, q2, k2, q_off, k_off) -> Shape:
    """The shape of a packed batch: Q_t [H, total_q, d_t], K_t [kv_t, total_k,
    d_t], sequence b at rows [q_off[b], q_off[b+1]) and [k_off[b],
    k_off[b+1]) of every head."""
    for t in (q1, k1, q2, k2):
        if t.dim() != 3:
            raise ValueError("packed Q and K tensors must be [H, N, d]")
        if not t.is_contiguous():
            raise ValueError("Q and K tensors must be contiguous")
        if t.dtype != q1.dtype:
            raise ValueError("Q1, K1, Q2, K2 must share one dtype")
        if t.device != q1.device:
            raise ValueError("Q1, K1, Q2, K2 must be on one device")
    if k_off is None or len(q_off) != len(k_off) or len(q_off) < 2:
        raise ValueError("q_off and k_off need B + 1 offsets each")
    H, n_q, d1 = q1.shape
    kv1, n_k, _ = k1.shape
    kv2, _, d2 = k2.shape
    if (tuple(k1.shape) != (kv1, n_k, d1) or tuple(q2.shape) != (H, n_q, d2) or tuple(k2.shape) != (kv2, n_k, d2)
            or H % kv1 or H % kv2):
        raise ValueError("inconsistent Q/K shapes")
    shp = make_shape(len(q_off) - 1, H, n_q, n_k, d1, d2, q1.dtype, 0 if kv1 == H else kv1, 0 if kv2 == H else kv2)
    return shp.set_offsets(q_off, k_off)


class _Layout:
    """The shapes of a call's tensors: [B, H, n_q] per-row vectors and
    [B, heads, n, d] gradients, or, for a packed batch, the same without the
    batch dimension."""

    def __init__(self, q1, k1, q2, k2, q_len=None, k_len=None, q_off=None, k_off=None):
        self.packed = q_off is not None or k_off is not None
        if self.packed:
            if q_len is not None or k_len is not None:
                raise ValueError("give lengths (padded batch) or offsets (packed batch), not both")
            self.shp = packed_shape_of(q1, k1, q2, k2, q_off, k_off)
        else:
            self.shp = shape_of(q1, k1, q2, k2).set_lengths(q_len, k_len)
        s = self.shp
        self.lead = () if self.packed else (s.B,)
        self.rows = self.lead + (s.H, s.n_q)

    def dq(self, d):
        return self.lead + (self.shp.H, self.shp.n_q, d)

    def dk(self, model, d):
        return self.lead + (_kv(self.shp, model), self.shp.n_k, d)


def _kv(shp: Shape, model: int) -> int:
    """Key heads of model 1 or 2."""
    kv = shp.kv_heads1 if model == 1 else shp.kv_heads2
    return kv if kv > 0 else shp.H


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _check(status: int, what: str):
    if status != OK:
        raise StreamKLError(status, what, _lib().streamkl_last_hip_error())


def _check_out(t, shape, device, what):
    """A caller-supplied output: fp32, contiguous, on the inputs' device, of the
    exact shape the library writes (it sees only a pointer)."""
    if t is None:
        raise ValueError(f"{what}: missing output tensor")
    if (t.dtype != torch.float32 or not t.is_contiguous() or t.device != device
            or tuple(t.shape) != tuple(shape)):
        raise ValueError(f"{what} must be a contiguous fp32 tensor of shape {tuple(shape)} on {device}, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")


def _check_rows(t, shp: Shape, device, what):
    """A per-row input vector: contiguous fp32 [B, H, n_q] ([H, n_q] for a
    packed batch) on the device."""
    rows = shp.H * shp.n_q * (1 if shp.q_off else shp.B)
    if t.dtype != torch.float32 or not t.is_contiguous() or t.numel() != rows or t.device != device:
        raise ValueError(f"{what} must be contiguous fp32 with one value per query row ([B, H, n_q], or [H, n_q] "
                         f"packed) on {device}")


def _bytes(n: int, what: str) -> int:
    if n == INVALID_BYTES:
        raise ValueError(f"{what}: invalid shape or launch options")
    return n


def _workspace(workspace, need: int, device):
    """The caller's workspace if it is a large enough device tensor, else a new one."""
    if workspace is not None:
        if workspace.device != device or not workspace.is_contiguous():
            raise ValueError(f"workspace must be a contiguous tensor on {device}")
        if workspace.numel() * workspace.element_size() >= need:
            return workspace
    return torch.empty(need, dtype=torch.uint8, device=device)


def fwd_plan(shape: Shape, causal: bool, num_splits: int = 0, with_workspace: bool = True) -> int:
    """Key-split count the forward would use."""
    lib = _lib()
    ln = Launch(num_splits, 0, None, 0)
    if with_workspace:
        ln.workspace_bytes = lib.streamkl_fwd_workspace_bytes(ctypes.byref(shape), int(causal), ctypes.byref(ln))
        ln.workspace = 16 if ln.workspace_bytes else None  # placeholder address, never dereferenced by the plan
    return lib.streamkl_fwd_plan(ctypes.byref(shape), int(causal), ctypes.byref(ln))


def fwd_workspace_bytes(shape: Shape, causal: bool, num_splits: int = 0) -> int:
    ln = Launch(num_splits, 0, None, 0)
    return _bytes(_lib().streamkl_fwd_workspace_bytes(ctypes.byref(shape), int(causal), ctypes.byref(ln)),
                  "streamkl_fwd_workspace_bytes")


def fwd_loss_workspace_bytes(shape: Shape, causal: bool, num_splits: int = 0) -> int:
    ln = Launch(num_splits, 0, None, 0)
    return _bytes(_lib().streamkl_fwd_loss_workspace_bytes(ctypes.byref(shape), int(causal), ctypes.byref(ln)),
                  "streamkl_fwd_loss_workspace_bytes")


def bwd_workspace_bytes(shape: Shape, causal: bool, setting: int, bwd_mode: int = BWD_AUTO) -> int:
    ln = Launch(0, bwd_mode, None, 0)
    return _bytes(_lib().streamkl_bwd_workspace_bytes(ctypes.byref(shape), int(causal), int(setting),
                                                      ctypes.byref(ln)), "streamkl_bwd_workspace_bytes")


def bwd_plan(shape: Shape, causal: bool, setting: int, bwd_mode: int = BWD_AUTO) -> int:
    ln = Launch(0, bwd_mode, None, 0)
    return _lib().streamkl_bwd_plan(ctypes.byref(shape), int(causal), int(setting), ctypes.byref(ln))


def streamkl_fwd(q1, k1, q2, k2, causal: bool, scale1: float = 0.0, scale2: float = 0.0,
                 num_splits: int = 0, out=None, workspace=None, q_len=None, k_len=None, q_off=None, k_off=None):
    """Forward: returns (kl, lse1, lse2), fp32 [B, H, n_q].

    num_splits: 0 = library's choice, 1 = no key split, k = k key splits.
    out: optional preallocated (kl, lse1, lse2).  workspace: optional uint8
    device tensor (allocated here when a split needs one and none is given).
    q_len, k_len: ragged batch in padded [B, H, N, d] tensors.  q_off, k_off:
    packed batch (B + 1 row offsets each) in [H, N, d] tensors; the outputs
    are then [H, n_q].
    """
    lay = _Layout(q1, k1, q2, k2, q_len, k_len, q_off, k_off)
    shp = lay.shp
    dev = q1.device
    rows = lay.rows
    if out is None:
        kw = dict(device=dev, dtype=torch.float32)
        out = tuple(torch.empty(rows, **kw) for _ in range(3))
    for t, n in zip(out, ("kl", "lse1", "lse2")):
        _check_out(t, rows, dev, f"out {n}")
    kl, lse1, lse2 = out
    ln = Launch(num_splits, 0, None, 0)
    need = _bytes(_lib().streamkl_fwd_workspace_bytes(ctypes.byref(shp), int(causal), ctypes.byref(ln)),
                  "streamkl_fwd")
    if need:
        workspace = _workspace(workspace, need, dev)
        ln.workspace = workspace.data_ptr()
        ln.workspace_bytes = workspace.numel() * workspace.element_size()
    st = _lib().streamkl_fwd(q1.data_ptr(), k1.data_ptr(), q2.data_ptr(), k2.data_ptr(), int(causal),
                             float(scale1), float(scale2), kl.data_ptr(), lse1.data_ptr(), lse2.data_ptr(),
                             ctypes.byref(shp), ctypes.byref(ln), _stream(dev))
    _check(st, "streamkl_fwd")
    return kl, lse1, lse2


def streamkl_fwd_loss(q1, k1, q2, k2, causal: bool, weights=None, scale1: float = 0.0, scale2: float = 0.0,
                      num_splits: int = 0, out=None, workspace=None, q_len=None, k_len=None, q_off=None,
                      k_off=None):
    """Forward with the loss fused into its epilogue: returns (kl, lse1, lse2, loss).

    loss is a 0-dim fp32 tensor: sum_i weights_i KL_i over every query row, or
    the mean KL over the rows when weights is None (bitwise repeatable).
    out: optional preallocated (kl, lse1, lse2, loss).  Batches as streamkl_fwd.
    """
    lay = _Layout(q1, k1, q2, k2, q_len, k_len, q_off, k_off)
    shp = lay.shp
    dev = q1.device
    rows = lay.rows
    if out is None:
        kw = dict(device=dev, dtype=torch.float32)
        out = tuple(torch.empty(rows, **kw) for _ in range(3)) + (torch.empty((), **kw),)
    for t, n in zip(out[:3], ("kl", "lse1", "lse2")):
        _check_out(t, rows, dev, f"out {n}")
    _check_out(out[3], (), dev, "out loss")
    if weights is not None:
        _check_rows(weights, shp, dev, "weights")
    kl, lse1, lse2, loss = out
    ln = Launch(num_splits, 0, None, 0)
    need = _bytes(_lib().streamkl_fwd_loss_workspace_bytes(ctypes.byref(shp), int(causal), ctypes.byref(ln)),
                  "streamkl_fwd_loss")
    workspace = _workspace(workspace, need, dev)
    ln.workspace = workspace.data_ptr()
    ln.workspace_bytes = workspace.numel() * workspace.element_size()
    st = _lib().streamkl_fwd_loss(q1.data_ptr(), k1.data_ptr(), q2.data_ptr(), k2.data_ptr(), int(causal),
                                  float(scale1), float(scale2), weights.data_ptr() if weights is not None else None,
                                  kl.data_ptr(), lse1.data_ptr(), lse2.data_ptr(), loss.data_ptr(),
                                  ctypes.byref(shp), ctypes.byref(ln), _stream(dev))
    _check(st, "streamkl_fwd_loss")
    return kl, lse1, lse2, loss


def streamkl_bwd(setting: int, q1, k1, q2, k2, causal: bool, kl, lse1, lse2, d_kl,
                 scale1: float = 0.0, scale2: float = 0.0, bwd_mode: int = BWD_AUTO, out=None,
                 q_len=None, k_len=None, q_off=None, k_off=None):
    """Backward: returns (dQ, dK) in fp32 for the trained model.

    setting 1 -> (dQ2, dK2) with P1 fixed; setting 2 -> (dQ1, dK1) with P2 fixed.
    q_len, k_len or q_off, k_off: the batch as given to the forward.
    """
    lay = _Layout(q1, k1, q2, k2, q_len, k_len, q_off, k_off)
    shp = lay.shp
    dev = q1.device
    ds = shp.d2 if setting == 1 else shp.d1
    model = 2 if setting == 1 else 1
    if out is None:
        kw = dict(device=dev, dtype=torch.float32)
        out = (None if bwd_mode == BWD_DK_ONLY else torch.empty(lay.dq(ds), **kw),
               None if bwd_mode == BWD_DQ_ONLY else torch.empty(lay.dk(model, ds), **kw))
    dq, dk = out
    if bwd_mode != BWD_DK_ONLY:
        _check_out(dq, lay.dq(ds), dev, "out dQ")
    if bwd_mode != BWD_DQ_ONLY:
        _check_out(dk, lay.dk(model, ds), dev, "out dK")
    for t, n in zip((lse1, lse2, d_kl, kl), ("lse1", "lse2", "d_kl", "kl")):
        if t is not None:
            _check_rows(t, shp, dev, n)
    ln = Launch(0, bwd_mode, None, 0)
    st = _lib().streamkl_bwd(int(setting), q1.data_ptr(), k1.data_ptr(), q2.data_ptr(), k2.data_ptr(), int(causal),
                             float(scale1), float(scale2), kl.data_ptr() if kl is not None else None,
                             lse1.data_ptr(), lse2.data_ptr(), d_kl.data_ptr(),
                             dq.data_ptr() if dq is not None else None, dk.data_ptr() if dk is not None else None,
                             ctypes.byref(shp), ctypes.byref(ln), _stream(dev))
    _check(st, "streamkl_bwd")
    return dq, dk


def streamkl_bwd_joint(q1, k1, q2, k2, causal: bool, kl, lse1, lse2, d_kl,
                       scale1: float = 0.0, scale2: float = 0.0, bwd_mode: int = BWD_AUTO, out=None,
                       q_len=None, k_len=None, q_off=None, k_off=None):
    """Joint backward: returns (dQ1, dK1, dQ2, dK2) in fp32, the gradients to
    both models in one pass (equal to setting 2 and setting 1 of streamkl_bwd)."""
    lay = _Layout(q1, k1, q2, k2, q_len, k_len, q_off, k_off)
    shp = lay.shp
    dev = q1.device
    shapes = (lay.dq(shp.d1), lay.dk(1, shp.d1), lay.dq(shp.d2), lay.dk(2, shp.d2))
    if out is None:
        kw = dict(device=dev, dtype=torch.float32)
        nq = bwd_mode == BWD_DK_ONLY
        nk = bwd_mode == BWD_DQ_ONLY
        out = tuple(None if (nq and i % 2 == 0) or (nk and i % 2 == 1) else torch.empty(sh, **kw)
                    for i, sh in enumerate(shapes))
    for i, (t, want, n) in enumerate(zip(out, shapes, ("dQ1", "dK1", "dQ2", "dK2"))):
        if (bwd_mode == BWD_DK_ONLY and i % 2 == 0) or (bwd_mode == BWD_DQ_ONLY and i % 2 == 1):
            continue
        _check_out(t, want, dev, f"out {n}")
    for t, n in zip((kl, lse1, lse2, d_kl), ("kl", "lse1", "lse2", "d_kl")):
        _check_rows(t, shp, dev, n)
    ln = Launch(0, bwd_mode, None, 0)
    ptr = lambda t: t.data_ptr() if t is not None else None  # noqa: E731
    st = _lib().streamkl_bwd_joint(q1.data_ptr(), k1.data_ptr(), q2.data_ptr(), k2.data_ptr(), int(causal),
                                   float(scale1), float(scale2), kl.data_ptr(), lse1.data_ptr(), lse2.data_ptr(),
                                   d_kl.data_ptr(), *(ptr(t) for t in out), ctypes.byref(shp), ctypes.byref(ln),
                                   _stream(dev))
    _check(st, "streamkl_bwd_joint")
    return tuple(out)


def kl_loss(kl, weights=None, out=None):
    """sum_i w_i KL_i over every row of kl (the mean KL when weights is None),
    as a 0-dim fp32 tensor computed by the library (deterministic)."""
    if kl.dtype != torch.float32 or not kl.is_contiguous():
        raise ValueError("kl must be contiguous fp32")
    if weights is not None and (weights.dtype != torch.float32 or not weights.is_contiguous()
                                or weights.numel() != kl.numel() or weights.device != kl.device):
        raise ValueError("weights must be contiguous fp32 with one value per row of kl")
    if out is None:
        out = torch.empty((), device=kl.device, dtype=torch.float32)
    _check_out(out, (), kl.device, "out")
    st = _lib().streamkl_kl_loss(kl.data_ptr(), weights.data_ptr() if weights is not None else None,
                                 kl.numel(), out.data_ptr(), _stream(kl.device))
    _check(st, "streamkl_kl_loss")
    return out


def _kl_input_grads(ctx, g):
    """Gradients of sum_i g_i KL_i to Q1, K1, Q2, K2 (those that need them):
    setting 1 for the student side, setting 2 for the teacher side, the
    joint backward for both."""
    q1, k1, q2, k2, kl, lse1, lse2 = ctx.saved_tensors[:7]
    g = g.contiguous().to(torch.float32)
    grads = [None, None, None, None]
    teacher = ctx.needs_input_grad[0] or ctx.needs_input_grad[1]
    student = ctx.needs_input_grad[2] or ctx.needs_input_grad[3]
    if teacher and student:
        dq1, dk1, dq2, dk2 = streamkl_bwd_joint(q1, k1, q2, k2, ctx.causal, kl, lse1, lse2, g, ctx.scale1,
                                                ctx.scale2, ctx.bwd_mode, **ctx.lens)
        return [dq1.to(q1.dtype), dk1.to(k1.dtype), dq2.to(q2.dtype), dk2.to(k2.dtype)]
    if student:
        dq2, dk2 = streamkl_bwd(1, q1, k1, q2, k2, ctx.causal, kl, lse1, lse2, g, ctx.scale1, ctx.scale2,
                                ctx.bwd_mode, **ctx.lens)
        grads[2], grads[3] = dq2.to(q2.dtype), dk2.to(k2.dtype)
    if teacher:
        dq1, dk1 = streamkl_bwd(2, q1, k1, q2, k2, ctx.causal, kl, lse1, lse2, g, ctx.scale1, ctx.scale2,
                                ctx.bwd_mode, **ctx.lens)
        grads[0], grads[1] = dq1.to(q1.dtype), dk1.to(k1.dtype)
    return grads


class _KLFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q1, k1, q2, k2, causal, scale1, scale2, bwd_mode, q_len, k_len, q_off, k_off):
        ctx.lens = dict(q_len=q_len, k_len=k_len, q_off=q_off, k_off=k_off)
        kl, lse1, lse2 = streamkl_fwd(q1, k1, q2, k2, causal, scale1, scale2, **ctx.lens)
        ctx.save_for_backward(q1, k1, q2, k2, kl, lse1, lse2)
        ctx.causal, ctx.scale1, ctx.scale2, ctx.bwd_mode = causal, scale1, scale2, bwd_mode
        return kl

    @staticmethod
    def backward(ctx, g):
        return (*_kl_input_grads(ctx, g), None, None, None, None, None, None, None, None)


class _KLLossFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q1, k1, q2, k2, weights, causal, scale1, scale2, bwd_mode, q_len, k_len, q_off, k_off):
        ctx.lens = dict(q_len=q_len, k_len=k_len, q_off=q_off, k_off=k_off)
        kl, lse1, lse2, loss = streamkl_fwd_loss(q1, k1, q2, k2, causal, weights, scale1, scale2, **ctx.lens)
        ctx.save_for_backward(q1, k1, q2, k2, kl, lse1, lse2, weights)
        ctx.causal, ctx.scale1, ctx.scale2, ctx.bwd_mode = causal, scale1, scale2, bwd_mode
        # the rows the mean counts: a packed batch has no padding
        H = kl.shape[-2]
        ctx.rows = kl.numel() if q_len is None else H * sum(int(x) for x in q_len)
        return loss

    @staticmethod
    def backward(ctx, gl):
        kl, weights = ctx.saved_tensors[4], ctx.saved_tensors[7]
        gl = gl.to(torch.float32)
        # d loss / d KL_i: w_i, or 1 / rows for the mean over the rows counted
        if weights is not None:
            g = weights * gl
        else:
            g = torch.empty_like(kl).fill_(1.0 / max(ctx.rows, 1)).mul_(gl)
        grad_w = kl * gl if ctx.needs_input_grad[4] else None
        return (*_kl_input_grads(ctx, g), grad_w, None, None, None, None, None, None, None, None)


def attention_kl(q1, k1, q2, k2, causal: bool = False, scale1: float = 0.0, scale2: float = 0.0,
                 bwd_mode: int = BWD_AUTO, q_len=None, k_len=None, q_off=None, k_off=None):
    """Per-row KL(P1 || P2) as an autograd function (gradients by streamkl_bwd).

    Gradients flow to whichever of (Q1, K1) / (Q2, K2) require grad: the
    student side uses setting 1 (teacher distribution held fixed), the
    teacher side setting 2 (student distribution held fixed), and both
    sides together the joint backward.  q_len, k_len: per batch element
    lengths of a ragged batch in padded tensors (padded rows give 0);
    q_off, k_off: row offsets of a packed batch in [H, N, d] tensors.
    """
    return _KLFunction.apply(q1, k1, q2, k2, causal, scale1, scale2, bwd_mode, q_len, k_len, q_off, k_off)


def attention_kl_loss(q1, k1, q2, k2, causal: bool = False, weights=None, scale1: float = 0.0,
                      scale2: float = 0.0, bwd_mode: int = BWD_AUTO, q_len=None, k_len=None, q_off=None,
                      k_off=None):
    """The distillation loss sum_i w_i KL_i (weights: fp32 [B, H, N_Q]), or the
    mean KL over the query rows (ragged batches: each element's rows), as a
    0-dim autograd tensor.  The forward forms it in its epilogue
    (streamkl_fwd_loss: no second pass over the KL, bitwise repeatable); the
    backward feeds d loss / d KL_i = w_i (or 1 / rows) to the kernels as
    attention_kl does, and gives weights the gradient KL_i when they
    require one."""
    return _KLLossFunction.apply(q1, k1, q2, k2, weights, causal, scale1, scale2, bwd_mode, q_len, k_len, q_off,
                                 k_off)
