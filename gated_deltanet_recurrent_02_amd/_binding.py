"""ctypes binding of libgdn.so (include/gdn.h): argument marshalling only.

Every function takes torch tensors on a HIP device, checks dtypes, shapes and contiguity,
and passes raw pointers plus torch's current stream to the C ABI; all arithmetic runs in the
library's kernels. There is no fallback: if libgdn.so is missing or fails to load, the first
call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

LIBRARY = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgdn.so")

GDN_OK, GDN_ERR_INVALID_ARGUMENT, GDN_ERR_UNSUPPORTED, GDN_ERR_OUT_OF_MEMORY, GDN_ERR_HIP = range(5)
GDN_F32, GDN_BF16, GDN_F16 = 0, 1, 2
_DTYPE_CODE = {torch.float32: GDN_F32, torch.bfloat16: GDN_BF16, torch.float16: GDN_F16}
_CODE_DTYPE = {GDN_F32: torch.float32, GDN_BF16: torch.bfloat16, GDN_F16: torch.float16}

# Every symbol include/gdn.h declares.
EXPORTS = ("gdn_state_alloc", "gdn_state_free", "gdn_decode_step", "gdn_decode_verify",
           "gdn_conv_gate_decode", "gdn_prefill_workspace_size", "gdn_prefill",
           "gdn_prefill_noalloc", "gdn_lowrank_decode_step", "gdn_status_string",
           "gdn_last_error")


class GDNError(RuntimeError):
    """A non-zero gdn_status; `.status` holds the code."""

    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


_lib = None


def lib():
    """The loaded library (loaded on first use). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY):
            raise ImportError(
                f"{LIBRARY} is missing: build it with `python -m gated_deltanet_recurrent_02_amd.build` "
                "(or __graft_entry__.build()); there is no fallback path")
        _lib = _declare(ctypes.CDLL(LIBRARY))
    return _lib


def _declare(L):
    P, i64, i32, f32, i = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_int
    L.gdn_state_alloc.argtypes = [i64, i32, i32, i32, i, ctypes.POINTER(P), ctypes.POINTER(ctypes.c_size_t)]
    L.gdn_state_alloc.restype = i
    L.gdn_state_free.argtypes = [P]
    L.gdn_state_free.restype = i
    L.gdn_decode_step.argtypes = [i64, i32, i32, i32, i32, P, P, P, i, P, P, P, i, P, f32, P]
    L.gdn_decode_step.restype = i
    L.gdn_decode_verify.argtypes = [i64, i32, i32, i32, i32, P, P, P, i, P, P, P, i, i32, P, P, P, P,
                                    P, P, f32, P]
    L.gdn_decode_verify.restype = i
    L.gdn_conv_gate_decode.argtypes = [i64, i32, i32, i32, i32, P, P, P, P, P, P, P, i, P, f32, f32, P]
    L.gdn_conv_gate_decode.restype = i
    L.gdn_prefill_workspace_size.argtypes = [i64, i32, i32, i32, i32, ctypes.POINTER(ctypes.c_size_t)]
    L.gdn_prefill_workspace_size.restype = i
    L.gdn_prefill.argtypes = [i64, i32, i32, i32, i32, P, P, P, i, P, P, P, i, P, f32, P,
                              ctypes.c_size_t, P]
    L.gdn_prefill.restype = i
    L.gdn_prefill_noalloc.argtypes = [i64, i32, i32, i32, i32, P, P, P, i, P, P, P, i, P, f32, P]
    L.gdn_prefill_noalloc.restype = i
    L.gdn_lowrank_decode_step.argtypes = [i64, i32, i32, i32, i32, i32, P, P, P, i, P, P, P, P, i,
                                          P, P, P, f32, P]
    L.gdn_lowrank_decode_step.restype = i
    L.gdn_status_string.argtypes = [i]
    L.gdn_status_string.restype = ctypes.c_char_p
    L.gdn_last_error.argtypes = []
    L.gdn_last_error.restype = ctypes.c_char_p
    return L


def check(status: int) -> None:
    """Raise GDNError with the library's message for a non-zero status."""
    if status != GDN_OK:
        L = lib()
        name = L.gdn_status_string(status).decode()
        raise GDNError(status, f"{name}: {L.gdn_last_error().decode()}")


def _ptr(t: torch.Tensor | None):
    return None if t is None else t.data_ptr()


# The current stream's raw handle without building a torch.cuda.Stream object (1.7 us per call
# from Python on the MI355X host; the raw accessor takes 0.1 us); torch builds without it take
# the public accessor.
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(dev: torch.device):
    if _raw_stream is not None:
        return _raw_stream(dev.index if dev.index is not None else torch.cuda.current_device())
    return torch.cuda.current_stream(dev).cuda_stream


def _need(t: torch.Tensor, name: str, shape: tuple, dtypes: tuple) -> None:
    # one combined test on the common path, the specific message only when it fails
    if (isinstance(t, torch.Tensor) and t.dtype in dtypes and t.shape == shape and t.is_cuda
            and t.is_contiguous()):
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a HIP device")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    raise ValueError(f"{name} must be contiguous")


_ACT = (torch.float32, torch.bfloat16, torch.float16)


def decode_step(q, k, v, alpha, beta, state, o=None, scale: float = 1.0):
    """gdn_decode_step on torch tensors; updates `state` in place and returns o.

    q, k [B,T,H,dk] and v [B,T,H,dv] share one dtype (fp32, bf16 or fp16); alpha, beta fp32
    [B,T,H]; state fp32, bf16 or fp16 [B,H,dv,dk]; o (optional) [B,T,H,dv] in the activation
    dtype."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    _need(q, "q", (B, T, H, dk), _ACT)
    _need(k, "k", (B, T, H, dk), (q.dtype,))
    _need(v, "v", (B, T, H, dv), (q.dtype,))
    _need(alpha, "alpha", (B, T, H), (torch.float32,))
    _need(beta, "beta", (B, T, H), (torch.float32,))
    _need(state, "state", (B, H, dv, dk), _ACT)
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=q.dtype, device=q.device)
    _need(o, "o", (B, T, H, dv), (q.dtype,))
    check(lib().gdn_decode_step(B, T, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _DTYPE_CODE[q.dtype],
                                _ptr(alpha), _ptr(beta), _ptr(state), _DTYPE_CODE[state.dtype],
                                _ptr(o), float(scale), _stream(q.device)))
    return o


def prefill_workspace_size(B: int, T: int, H: int, dk: int, dv: int) -> int:
    """gdn_prefill_workspace_size: bytes of workspace gdn_prefill needs for these sizes."""
    n = ctypes.c_size_t(0)
    check(lib().gdn_prefill_workspace_size(B, T, H, dk, dv, ctypes.byref(n)))
    return n.value


def prefill_workspace(q, v) -> torch.Tensor:
    """A uint8 device buffer of the workspace size for these q [B,T,H,dk] and v [..,dv]."""
    B, T, H, dk = q.shape
    n = prefill_workspace_size(B, T, H, dk, v.shape[-1])
    return torch.empty(max(n, 16), dtype=torch.uint8, device=q.device)


def prefill(q, k, v, alpha, beta, state, o=None, scale: float = 1.0, workspace=None):
    """gdn_prefill on torch tensors: the arguments and result of decode_step, computed in the
    chunked form; updates `state` in place and returns o. `workspace` (optional) is a device
    buffer of at least prefill_workspace_size(...) bytes; one is allocated when omitted."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    _need(q, "q", (B, T, H, dk), _ACT)
    _need(k, "k", (B, T, H, dk), (q.dtype,))
    _need(v, "v", (B, T, H, dv), (q.dtype,))
    _need(alpha, "alpha", (B, T, H), (torch.float32,))
    _need(beta, "beta", (B, T, H), (torch.float32,))
    _need(state, "state", (B, H, dv, dk), _ACT)
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=q.dtype, device=q.device)
    _need(o, "o", (B, T, H, dv), (q.dtype,))
    if workspace is None:
        workspace = prefill_workspace(q, v)
    if not (isinstance(workspace, torch.Tensor) and workspace.is_cuda and workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous device tensor")
    nbytes = workspace.numel() * workspace.element_size()
    check(lib().gdn_prefill(B, T, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _DTYPE_CODE[q.dtype],
                            _ptr(alpha), _ptr(beta), _ptr(state), _DTYPE_CODE[state.dtype],
                            _ptr(o), float(scale), _ptr(workspace), nbytes, _stream(q.device)))
    return o


def prefill_noalloc(q, k, v, alpha, beta, state, o, scale: float = 1.0):
    """gdn_prefill_noalloc on torch tensors: prefill() with the library's fixed device scratch
    instead of a workspace. Allocates nothing, so `o` must be given."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    _need(q, "q", (B, T, H, dk), _ACT)
    _need(k, "k", (B, T, H, dk), (q.dtype,))
    _need(v, "v", (B, T, H, dv), (q.dtype,))
    _need(alpha, "alpha", (B, T, H), (torch.float32,))
    _need(beta, "beta", (B, T, H), (torch.float32,))
    _need(state, "state", (B, H, dv, dk), _ACT)
    _need(o, "o", (B, T, H, dv), (q.dtype,))
    check(lib().gdn_prefill_noalloc(B, T, H, dk, dv, _ptr(q), _ptr(k), _ptr(v),
                                    _DTYPE_CODE[q.dtype], _ptr(alpha), _ptr(beta), _ptr(state),
                                    _DTYPE_CODE[state.dtype], _ptr(o), float(scale),
                                    _stream(q.device)))
    return o


def decode_verify(q, k, v, alpha, beta, state, prev=None, o=None, dk_out=None,
                  scale: float = 1.0):
    """gdn_decode_verify on torch tensors: commit the previous call's accepted prefix into
    `state`, then run the new tokens without storing the state after them.

    q, k, v, alpha, beta as decode_step (T may be 0 to commit only; pass tensors with T = 0).
    prev: None for the first call, else (n_prev int32 [B], k_prev [B,Tp,H,dk],
    alpha_prev [B,Tp,H], dk_prev fp32 [B,Tp,H,dv]) -- the previous call's k, alpha and dk_out
    and the accepted prefix lengths. Returns (o, dk_out)."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    _need(q, "q", (B, T, H, dk), _ACT)
    _need(k, "k", (B, T, H, dk), (q.dtype,))
    _need(v, "v", (B, T, H, dv), (q.dtype,))
    _need(alpha, "alpha", (B, T, H), (torch.float32,))
    _need(beta, "beta", (B, T, H), (torch.float32,))
    _need(state, "state", (B, H, dv, dk), _ACT)
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=q.dtype, device=q.device)
    if dk_out is None:
        dk_out = torch.empty((B, T, H, dv), dtype=torch.float32, device=q.device)
    _need(o, "o", (B, T, H, dv), (q.dtype,))
    _need(dk_out, "dk_out", (B, T, H, dv), (torch.float32,))
    Tp, n_prev, k_prev, alpha_prev, dk_prev = 0, None, None, None, None
    if prev is not None:
        n_prev, k_prev, alpha_prev, dk_prev = prev
        Tp = k_prev.shape[1]
        _need(n_prev, "n_prev", (B,), (torch.int32,))
        _need(k_prev, "k_prev", (B, Tp, H, dk), (q.dtype,))
        _need(alpha_prev, "alpha_prev", (B, Tp, H), (torch.float32,))
        _need(dk_prev, "dk_prev", (B, Tp, H, dv), (torch.float32,))
    check(lib().gdn_decode_verify(B, T, H, dk, dv, _ptr(q), _ptr(k), _ptr(v),
                                  _DTYPE_CODE[q.dtype], _ptr(alpha), _ptr(beta), _ptr(state),
                                  _DTYPE_CODE[state.dtype], Tp, _ptr(n_prev), _ptr(k_prev),
                                  _ptr(alpha_prev), _ptr(dk_prev), _ptr(o), _ptr(dk_out),
                                  float(scale), _stream(q.device)))
    return o, dk_out


def conv_gate_decode(qkv, conv_state, conv_w, conv_b, a_logit, b_logit, state, o=None,
                     scale: float = 1.0, l2_eps: float = 1e-6):
    """gdn_conv_gate_decode on torch tensors; updates `conv_state` and `state` in place and
    returns o (bf16 [B,T,H,dv]).

    qkv bf16 [B,T,C] with C = 3*H*D (blocks q | k | v); conv_state bf16 [B,C,3];
    conv_w fp32 [C,4]; conv_b fp32 [C] or None; a_logit, b_logit fp32 [B,T,H];
    state fp32, bf16 or fp16 [B,H,D,D]."""
    B, T, C = qkv.shape
    H = a_logit.shape[-1]
    D = state.shape[-1]
    _need(qkv, "qkv", (B, T, 3 * H * D), (torch.bfloat16,))
    _need(conv_state, "conv_state", (B, C, 3), (torch.bfloat16,))
    _need(conv_w, "conv_w", (C, 4), (torch.float32,))
    if conv_b is not None:
        _need(conv_b, "conv_b", (C,), (torch.float32,))
    _need(a_logit, "a_logit", (B, T, H), (torch.float32,))
    _need(b_logit, "b_logit", (B, T, H), (torch.float32,))
    _need(state, "state", (B, H, D, D), _ACT)
    if o is None:
        o = torch.empty((B, T, H, D), dtype=torch.bfloat16, device=qkv.device)
    _need(o, "o", (B, T, H, D), (torch.bfloat16,))
    check(lib().gdn_conv_gate_decode(B, T, H, D, D, _ptr(qkv), _ptr(conv_state), _ptr(conv_w),
                                     _ptr(conv_b), _ptr(a_logit), _ptr(b_logit), _ptr(state),
                                     _DTYPE_CODE[state.dtype], _ptr(o), float(scale),
                                     float(l2_eps), _stream(qkv.device)))
    return o


def lowrank_state(B: int, H: int, r: int, dk: int, dv: int, dtype: torch.dtype = torch.float32,
                  device="cuda") -> dict:
    """An empty sliding window (every slot zero, next slot 0) for lowrank_decode_step:
    U [B,H,r,dv] and K [B,H,r,dk] of `dtype`, c fp32 [B,H,r], pos int32 [B,H]."""
    return dict(U=torch.zeros((B, H, r, dv), dtype=dtype, device=device),
                K=torch.zeros((B, H, r, dk), dtype=dtype, device=device),
                c=torch.zeros((B, H, r), dtype=torch.float32, device=device),
                pos=torch.zeros((B, H), dtype=torch.int32, device=device))


def lowrank_decode_step(q, k, v, alpha, beta, U, K, c, pos, o=None, scale: float = 1.0):
    """gdn_lowrank_decode_step on torch tensors: T tokens on a sliding window of the last r
    writes; updates U, K, c and pos in place and returns o.

    q, k [B,T,H,dk], v [B,T,H,dv] (fp32, bf16 or fp16); alpha, beta fp32 [B,T,H];
    U [B,H,r,dv] and K [B,H,r,dk] in one state dtype (fp32, bf16 or fp16); c fp32 [B,H,r];
    pos int32 [B,H]; o (optional) [B,T,H,dv] in the activation dtype."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    r = U.shape[2] if U.dim() == 4 else -1
    _need(q, "q", (B, T, H, dk), _ACT)
    _need(k, "k", (B, T, H, dk), (q.dtype,))
    _need(v, "v", (B, T, H, dv), (q.dtype,))
    _need(alpha, "alpha", (B, T, H), (torch.float32,))
    _need(beta, "beta", (B, T, H), (torch.float32,))
    _need(U, "U", (B, H, r, dv), _ACT)
    _need(K, "K", (B, H, r, dk), (U.dtype,))
    _need(c, "c", (B, H, r), (torch.float32,))
    _need(pos, "pos", (B, H), (torch.int32,))
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=q.dtype, device=q.device)
    _need(o, "o", (B, T, H, dv), (q.dtype,))
    check(lib().gdn_lowrank_decode_step(B, T, H, dk, dv, r, _ptr(q), _ptr(k), _ptr(v),
                                        _DTYPE_CODE[q.dtype], _ptr(alpha), _ptr(beta), _ptr(U),
                                        _ptr(K), _DTYPE_CODE[U.dtype], _ptr(c), _ptr(pos),
                                        _ptr(o), float(scale), _stream(q.device)))
    return o


class StateBuffer:
    """A zero-filled state from gdn_state_alloc, freed with gdn_state_free when released.

    Exposes __cuda_array_interface__, so `torch.as_tensor(buf, device="cuda")` views it
    without a copy (the tensor keeps the buffer alive)."""

    def __init__(self, B: int, H: int, dk: int, dv: int, dtype: torch.dtype = torch.float32):
        self.shape = (B, H, dv, dk)
        self.dtype = dtype
        p = ctypes.c_void_p()
        n = ctypes.c_size_t()
        self._L = lib()
        check(self._L.gdn_state_alloc(B, H, dk, dv, _DTYPE_CODE[dtype], ctypes.byref(p),
                                      ctypes.byref(n)))
        self.ptr = p.value
        self.nbytes = n.value

    @property
    def __cuda_array_interface__(self):
        typestr = {torch.float32: "<f4", torch.float16: "<f2"}.get(self.dtype, "<V2")
        return {"shape": self.shape, "typestr": typestr, "data": (self.ptr, False),
                "version": 2, "strides": None}

    def tensor(self) -> torch.Tensor:
        """A torch view of the buffer (bf16 buffers are reinterpreted from 2-byte words)."""
        if self.dtype in (torch.float32, torch.float16):
            return torch.as_tensor(self, device="cuda")
        iface = {"shape": self.shape, "typestr": "<i2", "data": (self.ptr, False),
                 "version": 2, "strides": None}
        holder = type("_I16View", (), {"__cuda_array_interface__": iface, "_owner": self})()
        return torch.as_tensor(holder, device="cuda").view(torch.bfloat16)

    def free(self) -> None:
        if self.ptr:
            check(self._L.gdn_state_free(ctypes.c_void_p(self.ptr)))
            self.ptr = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def state_alloc(B: int, H: int, dk: int, dv: int, dtype: torch.dtype = torch.float32) -> StateBuffer:
    """gdn_state_alloc: a zero-filled [B,H,dv,dk] state owned by the returned object."""
    return StateBuffer(B, H, dk, dv, dtype)
