"""Helpers for comparing the GPU library with the fp64 oracle (used by the gpu-marked tests).

Error metric: for every (sequence, head), max |X - R| / max |R| over that head's tensor,
then the maximum over heads, so that a head with small values cannot hide behind a large one.
Bars (floating point):
  * fp32 state after all tokens: 1e-4; bf16-stored state: 2e-2 (its own rounding is 2^-8);
    fp16-stored state: 1e-3 (one rounding of 2^-11 relative, twice that for margin);
  * fp32 o: 1e-4 per token, relative to max(max|R_t|, 1e-3 max|R_head|): a token whose output
    is a small cancelling sum (alpha_t = 0 with k_t . q_t near 0, say) is held to 1e-7 of its
    head's largest output in absolute terms, since fp32 evaluation of a D-term dot product
    carries an absolute error of order sqrt(D) 2^-24 times its terms (the token-by-token kernel
    and the chunked form both show 6e-10 on such a token whose output is 8.5e-7 of a head at
    0.44);
  * bf16 o: 2e-2 per head, and elementwise |o - R| <= 2^-8 |R| + 1e-4 max|R_head| (one rounding
    to bf16 of an fp32 value that is itself within ~1e-6 of R); fp16 o: 1e-3 per head and
    elementwise |o - R| <= 2^-11 |R| + 1e-4 max|R_head|.
Integer/byte work (the conv state, a move of raw bf16 inputs) must match bit for bit.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import gated_deltanet_recurrent_02_amd as gdn
import oracle

TOL_STATE = {torch.float32: 1e-4, torch.bfloat16: 2e-2, torch.float16: 1e-3}
TOL_O_F32 = 1e-4
TOL_O_BF16 = 2e-2


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").double().numpy()


def head_rel_err(x: np.ndarray, ref: np.ndarray, nvec: int) -> float:
    """Max over heads of max|x - ref| / max|ref|; the last `nvec` axes form one head's tensor."""
    ax = tuple(range(x.ndim - nvec, x.ndim))
    d = np.abs(x - ref).max(axis=ax)
    n = np.abs(ref).max(axis=ax)
    if np.any(np.isnan(d)):
        return float("inf")
    return float(np.max(d / np.maximum(n, 1e-300)))


def check_state(state_gpu: np.ndarray, ref: np.ndarray, dtype: torch.dtype, what: str = "state"):
    e = head_rel_err(state_gpu, ref, 2)
    assert e <= TOL_STATE[dtype], f"{what}: per-head relative error {e:.3e} > {TOL_STATE[dtype]}"
    return e


def check_o(o_gpu: np.ndarray, ref: np.ndarray, dtype: torch.dtype, heads_axis_last: bool = True,
            extra: np.ndarray | float = 0.0):
    """o arrays [..., H, dv] (heads on the second-last axis). `extra` (broadcast to o) widens
    the elementwise bound of 16-bit outputs where an input is itself defined only up to a
    rounding (see stored_state_slack)."""
    if dtype == torch.float32:
        d = np.abs(o_gpu - ref).max(axis=-1)
        n = np.abs(ref).max(axis=-1)
        # The head's largest output: over the tokens (axis 1) of [B, T, H] maxima, else overall.
        head = n.max(axis=1, keepdims=True) if n.ndim == 3 else np.full_like(n, n.max())
        if np.any(np.isnan(d)):
            e = float("inf")
        else:
            e = float(np.max(d / np.maximum(np.maximum(n, 1e-3 * head), 1e-300)))
        assert e <= TOL_O_F32, f"o: per-token relative error {e:.3e} > {TOL_O_F32}"
        return e
    # ulp: one rounding relative to the value; sub: one rounding in the type's subnormal
    # range (half its smallest step), where the step is absolute
    tol, ulp, sub = ((TOL_O_BF16, 2.0 ** -8, 2.0 ** -134) if dtype == torch.bfloat16
                     else (1e-3, 2.0 ** -11, 2.0 ** -25))
    diff = np.abs(o_gpu - ref)
    if np.any(np.isnan(diff)):
        e = float("inf")
    else:
        d = np.maximum(diff - sub, 0.0).max(axis=-1)
        e = float(np.max(d / np.maximum(np.abs(ref).max(axis=-1), 1e-300)))
    assert e <= tol, f"o: per-head relative error {e:.3e} > {tol}"
    scale = np.abs(ref).max(axis=-1, keepdims=True)
    bound = ulp * np.abs(ref) + 1e-4 * scale + sub + extra
    bad = np.abs(o_gpu - ref) > bound
    assert not bad.any(), f"o: {int(bad.sum())} elements beyond one rounding to {dtype}"
    return e


def as_stored(S: np.ndarray, dtype) -> np.ndarray:
    """An fp64 state rounded to a storage type (round to nearest, ties to even, directly from
    fp64; the type's subnormals included), back in fp64: the state a call stores and the next
    call loads. dtype: torch.float32, torch.bfloat16 or torch.float16."""
    sig, emin = {torch.float32: (24, -126), torch.bfloat16: (8, -126), torch.float16: (11, -14)}[dtype]
    S = np.asarray(S, dtype=np.float64)
    _, e = np.frexp(S)                      # S = m 2^e, 0.5 <= |m| < 1
    quantum = np.ldexp(1.0, np.maximum(e - sig, emin - sig + 1))
    return np.rint(S / quantum) * quantum


def stored_state_slack(S_stored: np.ndarray, q: np.ndarray, dtype, flips: int = 2) -> np.ndarray:
    """Extra elementwise bound for o computed from a stored 16-bit state that the kernel rounds
    from its fp32 value and the reference from the exact one: near a rounding midpoint the two
    can land one unit apart. Allows `flips` such elements per state row: flips ulp(dtype)
    max_j |S[b, h, i, j]| max_j |q[b, t, h, j]|, shaped like o [B, T, H, dv]. 0 for fp32."""
    if dtype == torch.float32:
        return np.zeros(1)
    ulp = 2.0 ** -8 if dtype == torch.bfloat16 else 2.0 ** -11
    srow = np.abs(S_stored).max(axis=-1)            # [B, H, dv]
    qmax = np.abs(q).max(axis=-1)                   # [B, T, H]
    return flips * ulp * srow[:, None, :, :] * qmax[..., None]


def to_dev(x: dict, dev="cuda") -> dict:
    return {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}


def gpu_decode(x: dict, scale: float = 1.0):
    """Run gdn_decode_step on device copies of the inputs; returns (state_after, o) on device."""
    g = to_dev(x)
    o = gdn.decode_step(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["state"], scale=scale)
    torch.cuda.synchronize()
    return g["state"], o


def oracle_decode(x: dict, scale: float = 1.0, heads=None):
    """Oracle on all heads, or on the listed (b, h) pairs one by one (each pair becomes one
    sequence with one head). Returns (state [.., D, D], o [.., T, D]) with heads first when
    sampled, else the full [B,H,..] / [B,T,H,..] arrays."""
    if heads is None:
        return oracle.gdn_decode(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["alpha"]),
                                 f64(x["beta"]), f64(x["state"]), scale=scale)
    b, h = np.asarray(heads).T
    bt, ht = torch.as_tensor(b), torch.as_tensor(h)
    sel = lambda t: t[bt, :, ht]           # [n, T, D] or [n, T]
    q, k, v = (f64(sel(x[n]))[:, :, None] for n in ("q", "k", "v"))
    al, be = (f64(sel(x[n]))[:, :, None] for n in ("alpha", "beta"))
    S0 = f64(x["state"][bt, ht])[:, None]
    S, o = oracle.gdn_decode(q, k, v, al, be, S0, scale=scale)
    return S[:, 0], o[:, :, 0]


def oracle_decode_all(x: dict, scale: float = 1.0, workers: int = 0):
    """The oracle on every (b, h) head, the heads split over a thread pool (the C oracle runs
    outside the GIL). Returns (state [B,H,dv,dk], o [B,T,H,dv]) like oracle_decode(x)."""
    B, H = x["B"], x["H"]
    workers = workers or min(16, os.cpu_count() or 1)
    pairs = [(b, h) for b in range(B) for h in range(H)]
    groups = [g for g in np.array_split(np.asarray(pairs), workers) if len(g)]
    with ThreadPoolExecutor(len(groups)) as ex:
        parts = list(ex.map(lambda g: oracle_decode(x, scale, heads=[tuple(p) for p in g]), groups))
    S = np.concatenate([p[0] for p in parts])           # [B*H, dv, dk] in (b, h) order
    o = np.concatenate([p[1] for p in parts])           # [B*H, T, dv]
    T, dv = o.shape[1], o.shape[2]
    return (S.reshape(B, H, *S.shape[1:]),
            o.reshape(B, H, T, dv).transpose(0, 2, 1, 3))


def per_sequence(fn, B: int, workers: int = 0) -> list:
    """fn(b) for every sequence b on a thread pool (the C oracle runs outside the GIL);
    results in sequence order."""
    workers = workers or min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(min(workers, B)) as ex:
        return list(ex.map(fn, range(B)))


def oracle_prefix_all(x: dict, n, state: np.ndarray | None = None, workers: int = 0):
    """Per sequence b, the oracle's state after the first n[b] tokens of x (clamped to
    [0, T]), starting from `state` (fp64 [B,H,dv,dk]; x's state if None). Returns the fp64
    state [B,H,dv,dk]; sequences with an empty prefix keep their start state."""
    S0 = f64(x["state"]) if state is None else state
    T = x["T"]
    n = [min(max(int(v), 0), T) for v in n]

    def one(b):
        if n[b] == 0:
            return S0[b:b + 1]
        sl = slice(0, n[b])
        toks = [f64(x[m][b:b + 1, sl]) for m in ("q", "k", "v", "alpha", "beta")]
        return oracle.gdn_decode(*toks, S0[b:b + 1])[0]

    return np.concatenate(per_sequence(one, x["B"], workers))


def sample_heads(B: int, H: int, n: int, seed: int = 0):
    """The first and last head plus n random (b, h) pairs."""
    rng = np.random.default_rng(seed)
    pairs = {(0, 0), (B - 1, H - 1)}
    while len(pairs) < min(n + 2, B * H):
        pairs.add((int(rng.integers(B)), int(rng.integers(H))))
    return sorted(pairs)


# ----------------------------------------------------------------------------- low-rank window

LOWRANK_STATE = ("U", "K", "c", "pos")
TOL_C = 1e-5  # the weights are fp32 products of fp32 gates: a few roundings per token


def gpu_lowrank(x: dict, scale: float = 1.0):
    """gdn_lowrank_decode_step on device copies; returns (device dict with U, K, c, pos
    updated, o)."""
    g = to_dev(x)
    o = gdn.lowrank_decode_step(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["U"], g["K"],
                                g["c"], g["pos"], scale=scale)
    torch.cuda.synchronize()
    return g, o


def oracle_lowrank(x: dict, scale: float = 1.0, heads=None):
    """The oracle on every head, or on the listed (b, h) pairs one by one. Returns
    (U, K, c, pos, o) with the sampled heads first when `heads` is given ([n, ...] and o
    [n, T, dv]), else the full arrays."""
    if heads is None:
        return oracle.gdn_lowrank_decode(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["alpha"]),
                                         f64(x["beta"]), f64(x["U"]), f64(x["K"]), f64(x["c"]),
                                         x["pos"].numpy(), scale=scale)
    b, h = np.asarray(heads).T
    bt, ht = torch.as_tensor(b), torch.as_tensor(h)
    sel = lambda t: t[bt, :, ht]
    q, k, v = (f64(sel(x[n]))[:, :, None] for n in ("q", "k", "v"))
    al, be = (f64(sel(x[n]))[:, :, None] for n in ("alpha", "beta"))
    U, K, c = (f64(x[n][bt, ht])[:, None] for n in ("U", "K", "c"))
    pos = x["pos"][bt, ht].numpy()[:, None]
    U, K, c, pos, o = oracle.gdn_lowrank_decode(q, k, v, al, be, U, K, c, pos, scale=scale)
    return U[:, 0], K[:, 0], c[:, 0], pos[:, 0], o[:, :, 0]


def effective_state(U: np.ndarray, K: np.ndarray, c: np.ndarray) -> np.ndarray:
    """sum_i c_i U_i K_i^T over the slot axis (third from last of U), as one batched
    product (c-weighted U)^T K."""
    return np.matmul(np.swapaxes(U * c[..., None], -1, -2), K)


def check_lowrank(got: dict, o, ref, act: torch.dtype, sdt: torch.dtype):
    """got: U, K, c, pos (device or host tensors, same leading axes as ref); o [..., T, H, dv]
    or [n, T, dv]; ref = (U, K, c, pos, o) from the oracle. K is a copy of k rounded to the
    state dtype: bit-exact; pos: exact; U per head at the state bar; c at TOL_C; o at the
    activation bar; and the state the window stands for at the state bar."""
    U_ref, K_ref, c_ref, pos_ref, o_ref = ref
    U, K, c = (f64(got[n]) for n in ("U", "K", "c"))
    assert np.array_equal(got["pos"].cpu().numpy(), pos_ref), "pos"
    K_exp = f64(torch.from_numpy(K_ref).to(sdt))
    assert np.array_equal(K, K_exp), f"K: {int((K != K_exp).sum())} keys differ from k in {sdt}"
    e_c = head_rel_err(c, c_ref, 1)
    assert e_c <= TOL_C, f"c: per-head relative error {e_c:.3e} > {TOL_C}"
    check_state(U, U_ref, sdt, "U")
    check_state(effective_state(U, K, c), effective_state(U_ref, K_ref, c_ref), sdt,
                "effective state")
    return check_o(f64(o), o_ref, act)
