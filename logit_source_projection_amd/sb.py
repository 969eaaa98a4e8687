"""Thin Python binding of libsb (include/sb.h): argument marshalling only.

Every step of the head runs in libsb's HIP kernels.  PyTorch provides device
memory and the stream; this module builds the C descriptor from tensors,
allocates the workspace through torch when none is given, and raises
``SbError`` on a non-zero status.  A workspace allocated here is allocated on
the call's stream and recorded as used by it.  There is no fallback: if libsb.so is
missing, loading fails with an error.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsb.so")

SB_OK = 0
SB_ERR_NULL = -1
SB_ERR_SHAPE = -2
SB_ERR_LANES = -3
SB_ERR_ALIGN = -4
SB_ERR_WORKSPACE = -5
SB_ERR_UNSUPPORTED = -6
SB_ERR_HIP = -7

SB_SURF_TOKENS = 0
SB_SURF_LOGPROBS = 1
SB_SURF_LOGPROBS_FULL = 2
SB_SURF_FULL_LOGITS = 3

SB_MAX_LANES = 64

SB_RED_SUM = 0
SB_RED_PROD = 1
SB_RED_MIN = 2
SB_RED_MAX = 3
REDUCE_OPS = {"sum": SB_RED_SUM, "prod": SB_RED_PROD, "min": SB_RED_MIN, "max": SB_RED_MAX}

EXPORTS = ("sb_workspace_bytes", "sb_project_tokens", "sb_project_tokens_static",
           "sb_project_lane_results",
           "sb_project_logprobs", "sb_full_logits", "sb_partial_workspace_bytes",
           "sb_partial_complete", "sb_status_string")


class SbError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class sb_head_desc(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("H", ctypes.c_int32),
        ("V", ctypes.c_int32), ("k", ctypes.c_int32),
        ("lane_off", ctypes.POINTER(ctypes.c_int32)),
        ("x", ctypes.c_void_p), ("ldx", ctypes.c_int64),
        ("w", ctypes.POINTER(ctypes.c_void_p)), ("ldw", ctypes.c_int64),
    ]


class sb_partial_desc(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("N", ctypes.c_int32), ("k", ctypes.c_int32),
        ("lane_k", ctypes.POINTER(ctypes.c_int32)),
        ("x", ctypes.POINTER(ctypes.c_void_p)), ("ldx", ctypes.c_int64),
        ("w", ctypes.POINTER(ctypes.c_void_p)), ("ldw", ctypes.c_int64),
    ]


_lib = None


def lib():
    """The loaded libsb.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"libsb.so not found at {LIB_PATH}; build it first "
            "(python -c 'import __graft_entry__ as g; g.build()')")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(sb_head_desc)
    vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    L.sb_workspace_bytes.restype = sz
    L.sb_workspace_bytes.argtypes = [P, ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
    L.sb_project_tokens.restype = ctypes.c_int
    L.sb_project_tokens.argtypes = [P, vp, vp, sz, vp]
    L.sb_project_tokens_static.restype = ctypes.c_int
    L.sb_project_tokens_static.argtypes = [P, vp, vp]
    L.sb_project_lane_results.restype = ctypes.c_int
    L.sb_project_lane_results.argtypes = [P, vp, vp, vp, vp, sz, vp]
    L.sb_project_logprobs.restype = ctypes.c_int
    L.sb_project_logprobs.argtypes = [P, vp, vp, vp, vp, i64, vp, sz, vp]
    L.sb_full_logits.restype = ctypes.c_int
    L.sb_full_logits.argtypes = [P, vp, i64, vp, vp, sz, vp]
    PP = ctypes.POINTER(sb_partial_desc)
    L.sb_partial_workspace_bytes.restype = sz
    L.sb_partial_workspace_bytes.argtypes = [PP, ctypes.POINTER(ctypes.c_int)]
    L.sb_partial_complete.restype = ctypes.c_int
    L.sb_partial_complete.argtypes = [PP, ctypes.c_int, vp, i64, vp, sz, vp]
    L.sb_status_string.restype = ctypes.c_char_p
    L.sb_status_string.argtypes = [ctypes.c_int]
    _lib = L
    return L


def status_string(status):
    return lib().sb_status_string(int(status)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


# Argument checks of the binding: a host tensor, a wrong dtype or a strided
# layout the C ABI cannot express would otherwise reach a kernel as a raw
# pointer.  They raise before anything is enqueued.
def _device(t, name, dtype):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, not {t.dtype}")


def _vector(t, name, dtype, n):
    """A contiguous device buffer of at least n elements (None allowed)."""
    if t is None:
        return
    _device(t, name, dtype)
    if not t.is_contiguous() or t.numel() < n:
        raise ValueError(f"{name} must be contiguous with at least {n} elements")


def _matrix(t, name, dtype, rows, cols):
    """A [>= rows, >= cols] device matrix with unit column stride (None allowed)."""
    if t is None:
        return
    _device(t, name, dtype)
    if t.dim() != 2 or t.shape[0] < rows or t.shape[1] < cols or (
            t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError(f"{name} must be a [>= {rows}, >= {cols}] matrix with unit column stride")


def _operands(tensors, name):
    """The bf16 operands a descriptor was built from: on the device, rows
    with unit column stride."""
    for t in tensors:
        _device(t, name, torch.bfloat16)
        if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
            raise ValueError(f"{name} must be 2-D with unit column stride")


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


class Head:
    """Descriptor of a head: hidden rows x [B, H] (bf16) and the lane shards.

    ``w`` is either one [H, V] bf16 tensor (lanes are column ranges of it;
    every lane offset must then be a multiple of 8) or a list of k tensors,
    lane i of shape [H, V_i] with one common row stride.  ``lane_off`` holds
    the k+1 vocab offsets.  Raw values (pointers, strides) can be overridden
    to exercise the ABI's validation.
    """

    def __init__(self, x, w, lane_off, *, B=None, H=None, V=None, ldx=None,
                 ldw=None, x_ptr=None, w_ptrs=None):
        self.x = x
        self.w = w
        # built from tensors (checked on every call) or from raw pointers
        self.from_tensors = x_ptr is None and w_ptrs is None
        off = [int(o) for o in lane_off]
        self.lane_off = off
        k = len(off) - 1
        self._off = (ctypes.c_int32 * max(1, k + 1))(*off)
        if isinstance(w, (list, tuple)):
            ptrs = [t.data_ptr() for t in w]
            stride = w[0].stride(0) if len(w) else 0
        else:
            base = w.data_ptr()
            ptrs = [base + 2 * off[i] for i in range(k)]
            stride = w.stride(0)
        if w_ptrs is not None:
            ptrs = list(w_ptrs)
        self._w = (ctypes.c_void_p * max(1, len(ptrs)))(*ptrs)
        self.desc = sb_head_desc(
            B=x.shape[0] if B is None else B,
            H=x.shape[1] if H is None else H,
            V=off[-1] if V is None else V,
            k=k,
            lane_off=self._off,
            x=x.data_ptr() if x_ptr is None else x_ptr,
            ldx=x.stride(0) if ldx is None else ldx,
            w=self._w,
            ldw=stride if ldw is None else ldw)

    @property
    def B(self):
        return self.desc.B

    @property
    def V(self):
        return self.desc.V

    def ref(self):
        return ctypes.byref(self.desc)

    def check(self):
        if self.from_tensors:
            _operands([self.x], "x")
            _operands(self.w if isinstance(self.w, (list, tuple)) else [self.w], "w")


def sb_workspace_bytes(head, surface):
    st = ctypes.c_int(0)
    n = lib().sb_workspace_bytes(head.ref(), int(surface), ctypes.byref(st))
    if st.value != SB_OK:
        raise SbError(st.value, "sb_workspace_bytes")
    return int(n)


def workspace(head, surface, device="cuda"):
    """A workspace for `surface` (its contents on entry do not matter: every
    call clears what it relies on)."""
    n = sb_workspace_bytes(head, surface)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def _workspace(nbytes_fn, ws, device, stream):
    """The caller's workspace, or a temporary one allocated on the call's
    stream and marked as used by it, so that the caching allocator does not
    hand its memory to other work before the call's kernels are done."""
    if ws is not None:
        return ws
    s = _torch_stream(stream, device)
    with torch.cuda.stream(s):
        t = torch.empty(max(nbytes_fn(), 16), dtype=torch.uint8, device=device)
    t.record_stream(s)
    return t


def _torch_stream(stream, device):
    if stream is None:
        return torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream), device=device)


def _check(status, where):
    if status != SB_OK:
        raise SbError(status, where)


def sb_project_tokens(head, ids, ws=None, stream=None):
    """Token-only surface: ids (int32 [B], device) <- argmax token IDs."""
    head.check()
    _vector(ids, "ids", torch.int32, head.B)
    _vector(ws, "ws", torch.uint8, 0)
    ws = _workspace(lambda: sb_workspace_bytes(head, SB_SURF_TOKENS), ws, ids.device, stream)
    _check(lib().sb_project_tokens(head.ref(), _ptr(ids), _ptr(ws), ws.numel(),
                                   _stream(stream)), "sb_project_tokens")
    return ids


def sb_project_tokens_static(head, ids, stream=None):
    """Token-only surface with the library's static device scratch as the
    workspace (no allocation; SB_STATIC_SCRATCH_BYTES at most)."""
    head.check()
    _vector(ids, "ids", torch.int32, head.B)
    _check(lib().sb_project_tokens_static(head.ref(), _ptr(ids), _stream(stream)),
           "sb_project_tokens_static")
    return ids


SB_STATIC_SCRATCH_BYTES = 32 << 20


def sb_project_lane_results(head, ids, lane_ids=None, lane_max=None, ws=None, stream=None):
    """Token surface plus each lane's own result: lane_ids (int32 [B, k]) and
    lane_max (fp32 [B, k]) of every row, either optional."""
    head.check()
    k = head.desc.k
    _vector(ids, "ids", torch.int32, head.B)
    _vector(lane_ids, "lane_ids", torch.int32, head.B * k)
    _vector(lane_max, "lane_max", torch.float32, head.B * k)
    _vector(ws, "ws", torch.uint8, 0)
    ws = _workspace(lambda: sb_workspace_bytes(head, SB_SURF_TOKENS), ws, ids.device, stream)
    _check(lib().sb_project_lane_results(head.ref(), _ptr(ids), _ptr(lane_ids), _ptr(lane_max),
                                         _ptr(ws), ws.numel(), _stream(stream)),
           "sb_project_lane_results")
    return ids


def sb_project_logprobs(head, ids, lse, sel_lp=None, logprobs=None, ws=None,
                        stream=None):
    """Log-probability surface: ids, lse, optional sel_lp and complete
    fp32 log-probs [B, V] (row stride logprobs.stride(0))."""
    head.check()
    _vector(ids, "ids", torch.int32, head.B)
    _vector(lse, "lse", torch.float32, head.B)
    _vector(sel_lp, "sel_lp", torch.float32, head.B)
    _matrix(logprobs, "logprobs", torch.float32, head.B, head.V)
    _vector(ws, "ws", torch.uint8, 0)
    surf = SB_SURF_LOGPROBS_FULL if logprobs is not None else SB_SURF_LOGPROBS
    ws = _workspace(lambda: sb_workspace_bytes(head, surf), ws, ids.device, stream)
    ld = logprobs.stride(0) if logprobs is not None else 0
    _check(lib().sb_project_logprobs(head.ref(), _ptr(ids), _ptr(lse), _ptr(sel_lp),
                                     _ptr(logprobs), ld, _ptr(ws), ws.numel(),
                                     _stream(stream)), "sb_project_logprobs")
    return ids


def sb_full_logits(head, logits, ids=None, ws=None, stream=None):
    """Full-logit plan: logits fp32 [B, V] (row stride logits.stride(0)),
    optional ids."""
    head.check()
    _matrix(logits, "logits", torch.float32, head.B, head.V)
    _vector(ids, "ids", torch.int32, head.B)
    _vector(ws, "ws", torch.uint8, 0)
    ws = _workspace(lambda: sb_workspace_bytes(head, SB_SURF_FULL_LOGITS), ws, logits.device,
                    stream)
    _check(lib().sb_full_logits(head.ref(), _ptr(logits), logits.stride(0), _ptr(ids),
                                _ptr(ws), ws.numel(), _stream(stream)), "sb_full_logits")
    return logits


class Partial:
    """Descriptor of a row-parallel partial-completion boundary: k activation
    shards x[i] [B, K_i] (bf16, one common row stride) and weight blocks
    w[i] [K_i, N] (bf16, one common row stride).  Raw values can be
    overridden to exercise the ABI's validation."""

    def __init__(self, x, w, *, B=None, N=None, lane_k=None, ldx=None, ldw=None,
                 x_ptrs=None, w_ptrs=None):
        self.x, self.w = list(x), list(w)
        # built from tensors (checked on every call) or from raw pointers
        self.from_tensors = x_ptrs is None and w_ptrs is None
        Ks = [t.shape[1] for t in self.x]
        off = [0]
        for kk in Ks:
            off.append(off[-1] + kk)
        if lane_k is not None:
            off = [int(o) for o in lane_k]
        k = len(off) - 1
        self._off = (ctypes.c_int32 * max(1, k + 1))(*off)
        xp = [t.data_ptr() for t in self.x] if x_ptrs is None else list(x_ptrs)
        wp = [t.data_ptr() for t in self.w] if w_ptrs is None else list(w_ptrs)
        self._x = (ctypes.c_void_p * max(1, len(xp)))(*xp)
        self._w = (ctypes.c_void_p * max(1, len(wp)))(*wp)
        self.desc = sb_partial_desc(
            B=self.x[0].shape[0] if B is None else B,
            N=self.w[0].shape[1] if N is None else N,
            k=k, lane_k=self._off, x=self._x,
            ldx=self.x[0].stride(0) if ldx is None else ldx,
            w=self._w,
            ldw=self.w[0].stride(0) if ldw is None else ldw)

    @property
    def B(self):
        return self.desc.B

    @property
    def N(self):
        return self.desc.N

    def ref(self):
        return ctypes.byref(self.desc)

    def check(self):
        if self.from_tensors:
            _operands(self.x, "x")
            _operands(self.w, "w")


def sb_partial_workspace_bytes(part):
    st = ctypes.c_int(0)
    n = lib().sb_partial_workspace_bytes(part.ref(), ctypes.byref(st))
    if st.value != SB_OK:
        raise SbError(st.value, "sb_partial_workspace_bytes")
    return int(n)


def sb_partial_complete(part, op, out, ws=None, stream=None):
    """out (fp32 [B, N], row stride out.stride(0)) <- the registered
    reduction `op` ("sum", "prod", "min", "max" or an SB_RED_* code) of the
    lane partials."""
    code = REDUCE_OPS[op] if isinstance(op, str) else int(op)
    part.check()
    _matrix(out, "out", torch.float32, part.B, part.N)
    _vector(ws, "ws", torch.uint8, 0)
    ws = _workspace(lambda: sb_partial_workspace_bytes(part), ws, out.device, stream)
    _check(lib().sb_partial_complete(part.ref(), code, _ptr(out), out.stride(0), _ptr(ws),
                                     ws.numel(), _stream(stream)), "sb_partial_complete")
    return out


def to_device_bf16(bits, device="cuda"):
    """uint16 numpy bf16 bit patterns -> torch.bfloat16 tensor on device."""
    import numpy as np
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(device).view(torch.bfloat16)
