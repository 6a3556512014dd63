"""The C ABI on the CPU: libgdn.so loads, exports every symbol include/gdn.h declares, and
rejects invalid arguments on the host before any HIP call (fake device pointers are safe here
because validation fails before anything is enqueued)."""
import ctypes
import os
import re

import pytest
import torch

import gated_deltanet_recurrent_02_amd as gdn
from gated_deltanet_recurrent_02_amd import _binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")
INVALID, UNSUPPORTED, OOM, HIP = (bd.GDN_ERR_INVALID_ARGUMENT, bd.GDN_ERR_UNSUPPORTED,
                                  bd.GDN_ERR_OUT_OF_MEMORY, bd.GDN_ERR_HIP)
F32, BF16 = bd.GDN_F32, bd.GDN_BF16
BASE = 0x7F0000000000  # a fake, 256-byte aligned device address
MB = 1 << 20


def _gpu_visible():
    return torch.cuda.device_count() > 0


# Fake device pointers are only ever passed where no GPU is visible, so that a validation bug
# can never turn into a kernel launch on real hardware.
fake_ptrs = pytest.mark.skipif(_gpu_visible(), reason="passes fake device pointers")


def declared_functions():
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(gdn.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(bd.LIBRARY)
    for name in declared_functions():
        assert hasattr(L, name), name


def test_status_strings():
    L = gdn.lib()
    names = [L.gdn_status_string(i).decode() for i in range(5)]
    assert names == ["GDN_OK", "GDN_ERR_INVALID_ARGUMENT", "GDN_ERR_UNSUPPORTED",
                     "GDN_ERR_OUT_OF_MEMORY", "GDN_ERR_HIP"]
    assert L.gdn_status_string(99).decode() == "unknown"


def P(off=0):
    return ctypes.c_void_p(BASE + off)


def decode(B=2, T=1, H=4, dk=16, dv=16, q=None, k=None, v=None, act=F32, alpha=None, beta=None,
           state=None, sdt=F32, o=None, scale=1.0):
    """Call gdn_decode_step with disjoint fake buffers unless a pointer is given."""
    L = gdn.lib()
    q = P(0) if q is None else q
    k = P(16 * MB) if k is None else k
    v = P(32 * MB) if v is None else v
    alpha = P(48 * MB) if alpha is None else alpha
    beta = P(64 * MB) if beta is None else beta
    state = P(80 * MB) if state is None else state
    o = P(160 * MB) if o is None else o
    return L.gdn_decode_step(B, T, H, dk, dv, q, k, v, act, alpha, beta, state, sdt, o, scale, None)


def fused(B=2, T=2, H=4, D=16, qkv=None, cs=None, w=None, cb=None, a=None, b=None, state=None,
          sdt=F32, o=None, eps=1e-6):
    L = gdn.lib()
    qkv = P(0) if qkv is None else qkv
    cs = P(16 * MB) if cs is None else cs
    w = P(32 * MB) if w is None else w
    a = P(48 * MB) if a is None else a
    b = P(64 * MB) if b is None else b
    state = P(80 * MB) if state is None else state
    o = P(160 * MB) if o is None else o
    return L.gdn_conv_gate_decode(B, T, H, D, D, qkv, cs, w, cb, a, b, state, sdt, o, 1.0, eps, None)


def last_error():
    return gdn.lib().gdn_last_error().decode()


@pytest.mark.parametrize("kw,status,msg", [
    (dict(H=0), INVALID, "H must be"),
    (dict(B=-1), INVALID, "B and T"),
    (dict(T=-3), INVALID, "B and T"),
    (dict(dk=48, dv=48), UNSUPPORTED, "head dims"),
    (dict(dk=64, dv=128), UNSUPPORTED, "head dims"),
    (dict(dk=0, dv=0), INVALID, "dk and dv"),
    (dict(act=7), INVALID, "dtype"),
    (dict(sdt=-1), INVALID, "dtype"),
    (dict(q=ctypes.c_void_p(0)), INVALID, "q is NULL"),
    (dict(beta=ctypes.c_void_p(0)), INVALID, "beta is NULL"),
    (dict(q=P(8)), INVALID, "q is not 16-byte aligned"),
    (dict(state=P(80 * MB + 4)), INVALID, "state is not 16-byte aligned"),
    (dict(o=P(0)), INVALID, "o overlaps q"),
    (dict(o=P(80 * MB + 1024)), INVALID, "o overlaps state"),
    (dict(state=P(32 * MB)), INVALID, "state overlaps v"),
    (dict(B=1 << 26, H=32), INVALID, "B * H"),
    (dict(B=1 << 20, H=1 << 5), UNSUPPORTED, "B * H * 8 * dk"),   # 2^32 work-items
])
@fake_ptrs
def test_decode_step_rejects(kw, status, msg):
    assert decode(**kw) == status
    assert msg in last_error()


@fake_ptrs
def test_decode_step_empty_work_is_a_noop_even_with_null_pointers():
    L = gdn.lib()
    N = ctypes.c_void_p(0)
    for B, T in ((0, 1), (3, 0), (0, 0)):
        assert L.gdn_decode_step(B, T, 4, 128, 128, N, N, N, BF16, N, N, N, F32, N, 1.0, None) == 0
        assert last_error() == ""


@fake_ptrs
def test_adjacent_buffers_are_not_overlaps():
    # q holds B*T*H*dk fp32 = 2*1*4*16*4 = 512 bytes: o starting right after it passes
    # validation (and fails only at the launch, for lack of a device); 16 bytes earlier overlaps.
    assert decode(o=P(512), k=P(1 << 30), state=P(2 << 30)) == HIP
    assert decode(o=P(496)) == INVALID


@pytest.mark.parametrize("kw,status,msg", [
    (dict(H=0), INVALID, "H must be"),
    (dict(D=96), UNSUPPORTED, "head dims"),
    (dict(eps=-1.0), INVALID, "l2_eps"),
    (dict(eps=float("nan")), INVALID, "l2_eps"),
    (dict(cs=ctypes.c_void_p(0)), INVALID, "conv_state is NULL"),
    (dict(w=P(32 * MB + 8)), INVALID, "conv_w is not 16-byte aligned"),
    (dict(cb=P(200 * MB + 4)), INVALID, "conv_b is not 16-byte aligned"),
    (dict(cs=P(80 * MB)), INVALID, "conv_state overlaps state"),
    (dict(o=P(16 * MB)), INVALID, "o overlaps conv_state"),
    (dict(state=P(0)), INVALID, "state overlaps qkv"),
])
@fake_ptrs
def test_conv_gate_decode_rejects(kw, status, msg):
    assert fused(**kw) == status
    assert msg in last_error()


@fake_ptrs
def test_state_alloc_rejects():
    L = gdn.lib()
    p = ctypes.c_void_p()
    n = ctypes.c_size_t()
    assert L.gdn_state_alloc(4, 2, 16, 16, F32, None, None) == INVALID
    assert L.gdn_state_alloc(0, 2, 16, 16, F32, ctypes.byref(p), ctypes.byref(n)) == INVALID
    assert L.gdn_state_alloc(4, 2, 48, 48, F32, ctypes.byref(p), ctypes.byref(n)) == UNSUPPORTED
    assert L.gdn_state_alloc(4, 2, 16, 16, 5, ctypes.byref(p), ctypes.byref(n)) == INVALID
    assert L.gdn_state_alloc(1 << 62, 1 << 20, 128, 128, F32, ctypes.byref(p), ctypes.byref(n)) == INVALID
    assert "overflow" in last_error()
    assert L.gdn_state_free(None) == 0


@fake_ptrs
def test_valid_calls_without_a_device_report_hip_errors():
    L = gdn.lib()
    p = ctypes.c_void_p()
    n = ctypes.c_size_t()
    assert L.gdn_state_alloc(4, 2, 16, 16, F32, ctypes.byref(p), ctypes.byref(n)) == HIP
    assert p.value is None and last_error().startswith("gdn_state_alloc")
    assert decode() == HIP
    assert "kernel launch" in last_error()


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(bd, "_lib", None)
    monkeypatch.setattr(bd, "LIBRARY", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError, match="no fallback"):
        bd.lib()


def test_binding_rejects_cpu_tensors():
    q = torch.zeros(1, 1, 1, 16)
    with pytest.raises(ValueError, match="HIP device"):
        gdn.decode_step(q, q, q, torch.zeros(1, 1, 1), torch.zeros(1, 1, 1), torch.zeros(1, 1, 16, 16))


def verify(B=2, T=2, H=4, D=16, Tp=2, n_prev=None, k_prev=None, a_prev=None, d_prev=None,
           o=None, dk_out=None, state=None, q=None):
    L = gdn.lib()
    q = P(0) if q is None else q
    state = P(80 * MB) if state is None else state
    n_prev = P(200 * MB) if n_prev is None else n_prev
    k_prev = P(210 * MB) if k_prev is None else k_prev
    a_prev = P(220 * MB) if a_prev is None else a_prev
    d_prev = P(230 * MB) if d_prev is None else d_prev
    o = P(160 * MB) if o is None else o
    dk_out = P(170 * MB) if dk_out is None else dk_out
    return L.gdn_decode_verify(B, T, H, D, D, q, P(16 * MB), P(32 * MB), F32, P(48 * MB),
                               P(64 * MB), state, F32, Tp, n_prev, k_prev, a_prev, d_prev, o,
                               dk_out, 1.0, None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(Tp=-1), INVALID, "Tp must be"),
    (dict(n_prev=ctypes.c_void_p(0)), INVALID, "n_prev is NULL"),
    (dict(d_prev=P(230 * MB + 4)), INVALID, "dk_prev is not 16-byte aligned"),
    (dict(dk_out=ctypes.c_void_p(0)), INVALID, "dk_out is NULL"),
    (dict(dk_out=P(160 * MB + 64)), INVALID, "o overlaps dk_out"),
    (dict(dk_out=P(230 * MB)), INVALID, "dk_out overlaps dk_prev"),
    (dict(state=P(210 * MB)), INVALID, "state overlaps k_prev"),
    (dict(D=48), UNSUPPORTED, "head dims"),
])
@fake_ptrs
def test_decode_verify_rejects(kw, status, msg):
    assert verify(**kw) == status
    assert msg in last_error()


@fake_ptrs
def test_decode_verify_empty_parts_may_be_null():
    N = ctypes.c_void_p(0)
    # nothing to commit and nothing new: a no-op even with every pointer NULL
    assert gdn.lib().gdn_decode_verify(2, 0, 4, 16, 16, N, N, N, F32, N, N, N, F32, 0, N, N, N, N,
                                       N, N, 1.0, None) == 0
    # commit only (T = 0): new-token pointers may be NULL; passes validation, fails at launch
    assert verify(T=0, q=N, o=N, dk_out=N) == HIP


def prefill(B=2, T=40, H=4, D=16, q=None, o=None, state=None, ws=None, ws_bytes=None, act=F32):
    """gdn_prefill with disjoint fake buffers; the workspace is exactly the required size."""
    L = gdn.lib()
    q = P(0) if q is None else q
    state = P(80 * MB) if state is None else state
    o = P(160 * MB) if o is None else o
    ws = P(200 * MB) if ws is None else ws
    if ws_bytes is None:
        try:
            ws_bytes = gdn.prefill_workspace_size(B, T, H, D, D)
        except gdn.GDNError:
            ws_bytes = 1 << 30
    return L.gdn_prefill(B, T, H, D, D, q, P(16 * MB), P(32 * MB), act, P(48 * MB), P(64 * MB),
                         state, F32, o, 1.0, ws, ws_bytes, None)


def test_prefill_workspace_size():
    # one record of 544 fp32 per (b, h, chunk of 16 tokens)
    assert gdn.prefill_workspace_size(4, 4096, 48, 128, 128) == 4 * 48 * 256 * 2176
    assert gdn.prefill_workspace_size(2, 17, 3, 16, 16) == 2 * 3 * 2 * 2176
    assert gdn.prefill_workspace_size(2, 16, 3, 64, 64) == 2 * 3 * 1 * 2176
    assert gdn.prefill_workspace_size(0, 16, 3, 64, 64) == 0
    assert gdn.prefill_workspace_size(2, 0, 3, 64, 64) == 0
    L = gdn.lib()
    n = ctypes.c_size_t(7)
    assert L.gdn_prefill_workspace_size(2, 16, 3, 48, 48, ctypes.byref(n)) == UNSUPPORTED
    assert L.gdn_prefill_workspace_size(2, 16, 3, 64, 64, None) == INVALID


@pytest.mark.parametrize("kw,status,msg", [
    (dict(H=0), INVALID, "H must be"),
    (dict(D=96), UNSUPPORTED, "head dims"),
    (dict(act=9), INVALID, "dtype"),
    (dict(ws=ctypes.c_void_p(0)), INVALID, "workspace is NULL"),
    (dict(ws=P(200 * MB + 8)), INVALID, "workspace is not 16-byte aligned"),
    (dict(ws_bytes=1000), INVALID, "needed"),
    (dict(ws=P(16 * MB)), INVALID, "workspace overlaps k"),
    (dict(o=P(200 * MB)), INVALID, "o overlaps workspace"),
    (dict(state=P(200 * MB)), INVALID, "state overlaps workspace"),
    (dict(B=1 << 20, H=1 << 5), UNSUPPORTED, "B * H * 8 * dk"),
    (dict(B=1 << 10, H=1 << 10, T=2048), UNSUPPORTED, "ceil(T / 16)"),  # 2^33 prep threads
    (dict(B=1 << 10, H=1 << 9, T=2032, ws_bytes=1000), INVALID, "needed"),  # 127 * 2^25: fits
])
@fake_ptrs
def test_prefill_rejects(kw, status, msg):
    assert prefill(**kw) == status
    assert msg in last_error()


@fake_ptrs
def test_prefill_empty_work_and_valid_call_without_device():
    N = ctypes.c_void_p(0)
    assert gdn.lib().gdn_prefill(0, 16, 4, 16, 16, N, N, N, F32, N, N, N, F32, N, 1.0, N, 0, None) == 0
    assert gdn.lib().gdn_prefill(2, 0, 4, 16, 16, N, N, N, F32, N, N, N, F32, N, 1.0, N, 0, None) == 0
    assert prefill() == HIP
    assert "kernel launch" in last_error()


def prefill_noalloc(B=2, T=40, H=4, D=16, q=None, o=None, state=None, act=F32):
    """gdn_prefill_noalloc with disjoint fake buffers."""
    q = P(0) if q is None else q
    state = P(80 * MB) if state is None else state
    o = P(160 * MB) if o is None else o
    return gdn.lib().gdn_prefill_noalloc(B, T, H, D, D, q, P(16 * MB), P(32 * MB), act, P(48 * MB),
                                         P(64 * MB), state, F32, o, 1.0, None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(H=0), INVALID, "H must be"),
    (dict(D=96), UNSUPPORTED, "head dims"),
    (dict(act=9), INVALID, "dtype"),
    (dict(q=ctypes.c_void_p(0)), INVALID, "q is NULL"),
    (dict(o=P(80 * MB)), INVALID, "o overlaps state"),
    (dict(state=P(16 * MB)), INVALID, "state overlaps k"),
    # 48 heads x 650 chunks x 2176 bytes = 67,891,200 > 64 MiB of fixed scratch
    (dict(B=1, H=48, T=10400, D=128), UNSUPPORTED, "exceed the fixed scratch"),
    (dict(B=4, H=48, T=4096, D=128), UNSUPPORTED, "exceed the fixed scratch"),
])
@fake_ptrs
def test_prefill_noalloc_rejects(kw, status, msg):
    assert prefill_noalloc(**kw) == status
    assert msg in last_error()


@fake_ptrs
def test_prefill_noalloc_empty_work_and_valid_calls_without_device():
    N = ctypes.c_void_p(0)
    L = gdn.lib()
    assert L.gdn_prefill_noalloc(0, 16, 4, 16, 16, N, N, N, F32, N, N, N, F32, N, 1.0, None) == 0
    assert L.gdn_prefill_noalloc(2, 0, 4, 16, 16, N, N, N, F32, N, N, N, F32, N, 1.0, None) == 0
    # within the limit (the largest call that fits: 30,840 records of 2176 bytes <= 64 MiB);
    # validation passes and the call fails only where it needs the device
    assert prefill_noalloc() == HIP
    GB = 1 << 30
    assert L.gdn_prefill_noalloc(1, 514 * 16, 60, 128, 128, P(0), P(GB), P(2 * GB), F32,
                                 P(3 * GB), P(3 * GB + 4 * MB), P(4 * GB), F32, P(5 * GB), 1.0,
                                 None) == HIP
    assert "gdn_prefill_noalloc" in last_error()


def lowrank(B=2, T=2, H=4, D=16, r=16, q=None, k=None, v=None, act=F32, alpha=None, beta=None,
            U=None, K=None, sdt=F32, c=None, pos=None, o=None):
    """gdn_lowrank_decode_step with disjoint fake buffers unless a pointer is given."""
    L = gdn.lib()
    q = P(0) if q is None else q
    k = P(16 * MB) if k is None else k
    v = P(32 * MB) if v is None else v
    alpha = P(48 * MB) if alpha is None else alpha
    beta = P(64 * MB) if beta is None else beta
    U = P(80 * MB) if U is None else U
    K = P(100 * MB) if K is None else K
    c = P(120 * MB) if c is None else c
    pos = P(130 * MB) if pos is None else pos
    o = P(160 * MB) if o is None else o
    return L.gdn_lowrank_decode_step(B, T, H, D, D, r, q, k, v, act, alpha, beta, U, K, sdt, c,
                                     pos, o, 1.0, None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(H=0), INVALID, "H must be"),
    (dict(D=96), UNSUPPORTED, "head dims"),
    (dict(act=5), INVALID, "dtype"),
    (dict(r=0), INVALID, "r must be"),
    (dict(r=12), UNSUPPORTED, "r in {8, 16, 32}"),
    (dict(r=64), UNSUPPORTED, "r in {8, 16, 32}"),
    (dict(c=ctypes.c_void_p(0)), INVALID, "c is NULL"),
    (dict(pos=P(130 * MB + 4)), INVALID, "pos is not 16-byte aligned"),
    (dict(o=P(100 * MB)), INVALID, "o overlaps K"),
    (dict(U=P(100 * MB)), INVALID, "U overlaps K"),
    (dict(K=P(16 * MB)), INVALID, "K overlaps k"),
    (dict(c=P(130 * MB)), INVALID, "c overlaps pos"),
    (dict(pos=P(48 * MB)), INVALID, "pos overlaps alpha"),
    (dict(B=1 << 20, H=1 << 5), UNSUPPORTED, "B * H * 8 * dk"),
])
@fake_ptrs
def test_lowrank_decode_step_rejects(kw, status, msg):
    assert lowrank(**kw) == status
    assert msg in last_error()


@fake_ptrs
def test_lowrank_empty_work_and_valid_call_without_device():
    N = ctypes.c_void_p(0)
    L = gdn.lib()
    for B, T in ((0, 1), (3, 0)):
        assert L.gdn_lowrank_decode_step(B, T, 4, 128, 128, 16, N, N, N, BF16, N, N, N, N, F32, N,
                                         N, N, 1.0, None) == 0
    # U holds B*H*r*D fp32 = 2*4*16*16*4 = 8 KiB: K right after it is valid
    assert lowrank(K=P(80 * MB + 8192)) == HIP
    assert lowrank(K=P(80 * MB + 8192 - 16)) == INVALID
    assert lowrank() == HIP
    assert "kernel launch" in last_error()
