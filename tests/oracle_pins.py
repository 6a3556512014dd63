"""Pins that tie the fp64 oracle to facts other than its own code.

Each pin takes an oracle library handle (``oracle.load()`` or a mutant build) and raises
``AssertionError`` when the fact does not hold. The facts come from the mathematics of the
step and from hand-worked values, never from re-running the oracle's own formula:

* hand-worked dyadic examples (``golden/gdn_d2_worked.json``), matched exactly;
* the literal product of (I - beta k k^T) factors, an independent algorithm (explicit d x d
  matrices multiplied with numpy), on the tiny workload;
* special cases with closed forms: identity gate, zero decay, delta rule writes v, pure decay;
* structure: the change per token is rank one along k; linearity in (S0, v); tokens compose;
  heads are independent;
* the conv prologue against ``numpy.convolve`` and scipy's logistic function, identity taps,
  the roll of the conv state, unit norm after L2 normalisation.

Reading cited throughout: "GDN tuning limits on Kunlun XPU", section 二 (背景) gives the chain
short conv (kernel 4) -> gating -> recurrent rank-1-plus-decay update of a per-head state.
"""
from __future__ import annotations

import json
import os

import numpy as np
from scipy.special import expit

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rand_inputs(rng, B, T, H, dk, dv, unit_k=True):
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    alpha = rng.uniform(0.05, 0.99, (B, T, H))
    beta = rng.uniform(0.05, 0.99, (B, T, H))
    S0 = rng.standard_normal((B, H, dv, dk)) * 0.5
    return q, k, v, alpha, beta, S0


# ----------------------------------------------------------------------------- recurrence


def pin_golden_worked(lib):
    """Hand-worked dyadic examples reproduce exactly."""
    with open(os.path.join(GOLDEN, "gdn_d2_worked.json")) as f:
        doc = json.load(f)
    for case in doc["cases"]:
        toks = case["tokens"]
        T = len(toks)
        q = np.array([[t["q"] for t in toks]], dtype=float)[:, :, None, :]
        k = np.array([[t["k"] for t in toks]], dtype=float)[:, :, None, :]
        v = np.array([[t["v"] for t in toks]], dtype=float)[:, :, None, :]
        al = np.array([[t["alpha"] for t in toks]], dtype=float)[:, :, None]
        be = np.array([[t["beta"] for t in toks]], dtype=float)[:, :, None]
        S0 = np.array(case["S0"], dtype=float)[None, None]
        S, o = oracle.gdn_decode(q, k, v, al, be, S0, lib=lib)
        assert np.array_equal(S[0, 0], np.array(case["S_final"], dtype=float)), case["name"]
        assert np.array_equal(o[0, :, 0, :], np.array(case["o"], dtype=float)), case["name"]
        assert o.shape == (1, T, 1, 2)


def closed_form_product(S0, q, k, v, alpha, beta):
    """S_T and every o_t for one head by explicit matrix products.

    S_t = (prod_{s<=t} alpha_s) S0 A_1..A_t + sum_{r<=t} (prod_{r<s<=t} alpha_s) beta_r v_r k_r^T A_{r+1}..A_t,
    A_s = I - beta_s k_s k_s^T; o_t = S_t q_t. Built from d x d matrices and numpy products,
    not from the per-row update the oracle uses."""
    T, dk = k.shape
    I = np.eye(dk)
    A = [I - beta[s] * np.outer(k[s], k[s]) for s in range(T)]
    outs = []
    for t in range(T):
        lead = np.prod(alpha[: t + 1])
        P = I.copy()
        for s in range(t + 1):
            P = P @ A[s]
        St = lead * (S0 @ P)
        for r in range(t + 1):
            Pr = I.copy()
            for s in range(r + 1, t + 1):
                Pr = Pr @ A[s]
            St = St + np.prod(alpha[r + 1: t + 1]) * beta[r] * (np.outer(v[r], k[r]) @ Pr)
        outs.append(St @ q[t])
    return St, np.array(outs)


def pin_closed_form(lib, B=1, H=2, D=16, T=8, zero_state=True, seed=0):
    """Oracle equals the literal product of (I - beta k k^T) factors, to ~1e-13."""
    rng = np.random.default_rng(seed)
    q, k, v, al, be, S0 = _rand_inputs(rng, B, T, H, D, D)
    if zero_state:
        S0[:] = 0.0
    S, o = oracle.gdn_decode(q, k, v, al, be, S0, lib=lib)
    for b in range(B):
        for h in range(H):
            Sx, ox = closed_form_product(S0[b, h], q[b, :, h], k[b, :, h], v[b, :, h],
                                         al[b, :, h], be[b, :, h])
            assert np.max(np.abs(S[b, h] - Sx)) <= 1e-12 * max(1.0, np.max(np.abs(Sx)))
            assert np.max(np.abs(o[b, :, h] - ox)) <= 1e-12 * max(1.0, np.max(np.abs(ox)))


def pin_identity_gate(lib, seed=1):
    """alpha = 1, beta = 0 leaves S bit-identical and reads o = S q."""
    rng = np.random.default_rng(seed)
    q, k, v, al, be, S0 = _rand_inputs(rng, 2, 3, 3, 8, 8)
    al[:] = 1.0
    be[:] = 0.0
    S, o = oracle.gdn_decode(q, k, v, al, be, S0, lib=lib)
    assert np.array_equal(S, S0)
    for t in range(3):
        ref = np.einsum("bhij,bhj->bhi", S0, q[:, t])
        assert np.max(np.abs(o[:, t] - ref)) <= 1e-13


def pin_zero_decay(lib, seed=2):
    """alpha = 0 forgets the past: S = beta v k^T and o = beta v (k . q)."""
    rng = np.random.default_rng(seed)
    q, k, v, al, be, S0 = _rand_inputs(rng, 1, 1, 4, 8, 8)
    al[:] = 0.0
    S, o = oracle.gdn_decode(q, k, v, al, be, S0, lib=lib)
    for h in range(4):
        ref = be[0, 0, h] * np.outer(v[0, 0, h], k[0, 0, h])
        assert np.max(np.abs(S[0, h] - ref)) <= 1e-14
        ref_o = be[0, 0, h] * v[0, 0, h] * np.dot(k[0, 0, h], q[0, 0, h])
        assert np.max(np.abs(o[0, 0, h] - ref_o)) <= 1e-14


def pin_writes_v(lib, seed=3):
    """alpha = beta = 1 with unit-norm k: the new state maps k to v (S k = v), whatever S0."""
    rng = np.random.default_rng(seed)
    q, k, v, al, be, S0 = _rand_inputs(rng, 1, 1, 3, 16, 16)
    al[:] = 1.0
    be[:] = 1.0
    S0 *= 10.0
    S, _ = oracle.gdn_decode(q, k, v, al, be, S0, lib=lib)
    for h in range(3):
        assert np.max(np.abs(S[0, h] @ k[0, 0, h] - v[0, 0, h])) <= 1e-12


def pin_pure_decay(lib, seed=4):
    """beta = 0: S_t = alpha_t S_{t-1}, so after T tokens S = (prod alpha) S0."""
    rng = np.random.default_rng(seed)
    q, k, v, al, be, S0 = _rand_inputs(rng, 1, 4, 2, 8, 8)
    be[:] = 0.0
    S, _ = oracle.gdn_decode(q, k, v, al, be, S0, lib=lib)
    for h in range(2):
        ref = np.prod(al[0, :, h]) * S0[0, h]
        assert np.max(np.abs(S[0, h] - ref)) <= 1e-14


def pin_rank_one(lib, seed=5):
    """S_t - alpha_t S_{t-1} has rank one and its rows are multiples of k_t (the rank-1
    update of the state named in the page's background section)."""
    rng = np.random.default_rng(seed)
    q, k, v, al, be, S0 = _rand_inputs(rng, 1, 1, 2, 16, 16)
    S, _ = oracle.gdn_decode(q, k, v, al, be, S0, lib=lib)
    for h in range(2):
        Dm = S[0, h] - al[0, 0, h] * S0[0, h]
        sv = np.linalg.svd(Dm, compute_uv=False)
        assert sv[1] <= 1e-12 * sv[0]
        kk = k[0, 0, h] / np.linalg.norm(k[0, 0, h])
        resid = Dm - np.outer(Dm @ kk, kk)
        assert np.max(np.abs(resid)) <= 1e-12 * max(1.0, np.max(np.abs(Dm)))


def pin_tokens_compose(lib, seed=6):
    """A T-token call equals T one-token calls, and a call split 3 + 2 resumes exactly."""
    rng = np.random.default_rng(seed)
    q, k, v, al, be, S0 = _rand_inputs(rng, 2, 5, 2, 8, 8)
    S, o = oracle.gdn_decode(q, k, v, al, be, S0, lib=lib)
    Sx = S0
    for t in range(5):
        sl = slice(t, t + 1)
        Sx, ot = oracle.gdn_decode(q[:, sl], k[:, sl], v[:, sl], al[:, sl], be[:, sl], Sx,
                                   lib=lib)
        assert np.array_equal(ot[:, 0], o[:, t])
    assert np.array_equal(Sx, S)
    S3, _ = oracle.gdn_decode(q[:, :3], k[:, :3], v[:, :3], al[:, :3], be[:, :3], S0, lib=lib)
    S5, o5 = oracle.gdn_decode(q[:, 3:], k[:, 3:], v[:, 3:], al[:, 3:], be[:, 3:], S3, lib=lib)
    assert np.array_equal(S5, S) and np.array_equal(o5, o[:, 3:])


def pin_head_independence(lib, seed=7):
    """Each (sequence, head) depends only on its own inputs: reversing the batch and heads
    reverses the outputs, and a single head run alone gives the same bits."""
    rng = np.random.default_rng(seed)
    q, k, v, al, be, S0 = _rand_inputs(rng, 3, 2, 4, 8, 8)
    S, o = oracle.gdn_decode(q, k, v, al, be, S0, lib=lib)
    fl = lambda a, ax: np.ascontiguousarray(np.flip(a, axis=ax))
    Sr, orr = oracle.gdn_decode(fl(fl(q, 0), 2), fl(fl(k, 0), 2), fl(fl(v, 0), 2),
                                fl(fl(al, 0), 2), fl(fl(be, 0), 2), fl(fl(S0, 0), 1), lib=lib)
    assert np.array_equal(fl(fl(Sr, 0), 1), S) and np.array_equal(fl(fl(orr, 0), 2), o)
    b, h = 2, 1
    S1, o1 = oracle.gdn_decode(q[b:b + 1, :, h:h + 1], k[b:b + 1, :, h:h + 1],
                               v[b:b + 1, :, h:h + 1], al[b:b + 1, :, h:h + 1],
                               be[b:b + 1, :, h:h + 1], S0[b:b + 1, h:h + 1], lib=lib)
    assert np.array_equal(S1[0, 0], S[b, h]) and np.array_equal(o1[0, :, 0], o[b, :, h])


def pin_linearity(lib, seed=8):
    """For fixed q, k, alpha, beta the map (S0, v) -> (S_T, o) is linear."""
    rng = np.random.default_rng(seed)
    q, k, va, al, be, Sa = _rand_inputs(rng, 1, 3, 2, 8, 8)
    vb = rng.standard_normal(va.shape)
    Sb = rng.standard_normal(Sa.shape)
    c = 0.37
    S1, o1 = oracle.gdn_decode(q, k, va, al, be, Sa, lib=lib)
    S2, o2 = oracle.gdn_decode(q, k, vb, al, be, Sb, lib=lib)
    S3, o3 = oracle.gdn_decode(q, k, va + c * vb, al, be, Sa + c * Sb, lib=lib)
    assert np.max(np.abs(S3 - (S1 + c * S2))) <= 1e-12
    assert np.max(np.abs(o3 - (o1 + c * o2))) <= 1e-12


def pin_scale(lib, seed=9):
    """The readout scale multiplies q only: o(scale) = scale * o(1), state unchanged."""
    rng = np.random.default_rng(seed)
    q, k, v, al, be, S0 = _rand_inputs(rng, 1, 2, 2, 8, 8)
    S1, o1 = oracle.gdn_decode(q, k, v, al, be, S0, scale=1.0, lib=lib)
    S2, o2 = oracle.gdn_decode(q, k, v, al, be, S0, scale=0.125, lib=lib)
    assert np.array_equal(S1, S2)
    assert np.max(np.abs(o2 - 0.125 * o1)) <= 1e-15


# ----------------------------------------------------------------------------- prologue


def _prologue_inputs(rng, B, T, H, D, bias=False):
    C = 3 * H * D
    x = rng.standard_normal((B, T, C))
    cs = rng.standard_normal((B, C, 3))
    w = rng.standard_normal((C, 4)) * 0.5
    cb = rng.standard_normal(C) * 0.1 if bias else None
    a = rng.standard_normal((B, T, H)) * 2
    b = rng.standard_normal((B, T, H)) * 2
    return x, cs, w, cb, a, b


def _silu(y):
    return y * expit(y)


def pin_conv_matches_numpy(lib, seed=10, bias=False):
    """Per channel, the pre-activation is numpy.convolve('valid') of (conv state | new inputs)
    with the reversed taps (tap 3 on the current input); v is its SiLU, and q, k are the SiLU
    outputs of the q and k channel blocks scaled to unit length."""
    rng = np.random.default_rng(seed)
    B, T, H, D = 2, 5, 3, 4
    x, cs, w, cb, a, b = _prologue_inputs(rng, B, T, H, D, bias=bias)
    q, k, v, al, be, cs_new = oracle.conv_gate(x, cs, w, cb, a, b, H, D, D, l2_eps=0.0, lib=lib)
    C = 3 * H * D
    y = np.zeros((B, T, C))
    for bb in range(B):
        for c in range(C):
            u = np.concatenate([cs[bb, c], x[bb, :, c]])
            y[bb, :, c] = np.convolve(u, w[c][::-1], mode="valid")
            if cb is not None:
                y[bb, :, c] += cb[c]
    s = _silu(y)
    sq = s[:, :, : H * D].reshape(B, T, H, D)
    sk = s[:, :, H * D: 2 * H * D].reshape(B, T, H, D)
    sv = s[:, :, 2 * H * D:].reshape(B, T, H, D)
    assert np.max(np.abs(v - sv)) <= 1e-13
    assert np.max(np.abs(q - sq / np.linalg.norm(sq, axis=-1, keepdims=True))) <= 1e-13
    assert np.max(np.abs(k - sk / np.linalg.norm(sk, axis=-1, keepdims=True))) <= 1e-13


def pin_conv_bias(lib):
    pin_conv_matches_numpy(lib, seed=11, bias=True)


def pin_conv_identity_taps(lib, seed=12):
    """Taps (0, 0, 0, 1) pass the current input through: v = SiLU(x_t) exactly."""
    rng = np.random.default_rng(seed)
    B, T, H, D = 1, 3, 2, 4
    x, cs, w, _, a, b = _prologue_inputs(rng, B, T, H, D)
    w[:] = 0.0
    w[:, 3] = 1.0
    _, _, v, _, _, _ = oracle.conv_gate(x, cs, w, None, a, b, H, D, D, lib=lib)
    xv = x[:, :, 2 * H * D:].reshape(B, T, H, D)
    assert np.max(np.abs(v - _silu(xv))) <= 1e-15
    w[:] = 0.0
    w[:, 0] = 1.0   # the oldest tap reads the cached input three tokens back
    _, _, v, _, _, _ = oracle.conv_gate(x, cs, w, None, a, b, H, D, D, lib=lib)
    cv = cs[:, 2 * H * D:, :]
    for t in range(T):
        assert np.max(np.abs(v[0, t].reshape(-1) - _silu(cv[0, :, t]))) <= 1e-15


def pin_conv_state_roll(lib, seed=13):
    """After T tokens the conv state holds the last three raw inputs, oldest first; for T < 3
    the oldest entries come from the previous state."""
    rng = np.random.default_rng(seed)
    for T in (1, 2, 3, 5):
        B, H, D = 2, 1, 4
        x, cs, w, _, a, b = _prologue_inputs(rng, B, T, H, D)
        *_, cs_new = oracle.conv_gate(x, cs, w, None, a, b, H, D, D, lib=lib)
        seq = np.concatenate([cs, np.transpose(x, (0, 2, 1))], axis=2)  # [B, C, 3 + T]
        assert np.array_equal(cs_new, seq[:, :, -3:]), T


def pin_unit_norm(lib, seed=14):
    """q and k come out with length sqrt(n / (n + eps)), n the squared length before scaling."""
    rng = np.random.default_rng(seed)
    B, T, H, D = 1, 2, 2, 8
    x, cs, w, _, a, b = _prologue_inputs(rng, B, T, H, D)
    for eps in (0.0, 1e-6, 0.5):
        q, k, *_ = oracle.conv_gate(x, cs, w, None, a, b, H, D, D, l2_eps=eps, lib=lib)
        q0, k0, *_ = oracle.conv_gate(x, cs, w, None, a, b, H, D, D, l2_eps=0.0, lib=lib)
        # q0 is a unit vector; q = q0 * sqrt(n) / sqrt(n + eps)
        assert np.max(np.abs(np.linalg.norm(q0, axis=-1) - 1.0)) <= 1e-14
        assert np.max(np.abs(np.linalg.norm(k0, axis=-1) - 1.0)) <= 1e-14
        rq = np.linalg.norm(q, axis=-1)
        assert np.all(rq <= 1.0 + 1e-14)
        if eps == 0.5:
            assert np.min(rq) < 1.0 - 1e-6


def pin_gates(lib, seed=15):
    """beta = logistic(b); alpha = exp(-softplus(a)) = 1 / (1 + e^a) = logistic(-a), checked
    against scipy's expit, including alpha(0) = beta(0) = 1/2 and extreme logits."""
    rng = np.random.default_rng(seed)
    B, T, H, D = 1, 4, 6, 2
    x, cs, w, _, a, b = _prologue_inputs(rng, B, T, H, D)
    a[0, 0] = [0.0, 50.0, -50.0, 800.0, -800.0, 3.0]
    b[0, 0] = [0.0, 50.0, -50.0, 800.0, -800.0, -3.0]
    _, _, _, al, be, _ = oracle.conv_gate(x, cs, w, None, a, b, H, D, D, lib=lib)
    assert al[0, 0, 0] == 0.5 and be[0, 0, 0] == 0.5
    assert np.all(np.isfinite(al)) and np.all(np.isfinite(be))
    assert np.all((al >= 0) & (al <= 1)) and np.all((be >= 0) & (be <= 1))
    np.testing.assert_allclose(be, expit(b), rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(al, expit(-a), rtol=1e-13, atol=1e-300)


def pin_fused_composes(lib, seed=16):
    """The fused entry point equals the prologue followed by the decode step."""
    rng = np.random.default_rng(seed)
    B, T, H, D = 2, 3, 2, 8
    x, cs, w, cb, a, b = _prologue_inputs(rng, B, T, H, D, bias=True)
    S0 = rng.standard_normal((B, H, D, D))
    q, k, v, al, be, cs1 = oracle.conv_gate(x, cs, w, cb, a, b, H, D, D, lib=lib)
    S1, o1 = oracle.gdn_decode(q, k, v, al, be, S0, scale=0.5, lib=lib)
    S2, o2, cs2 = oracle.gdn_conv_gate_decode(x, cs, w, cb, a, b, S0, H, D, D, scale=0.5,
                                              lib=lib)
    assert np.array_equal(S1, S2) and np.array_equal(o1, o2) and np.array_equal(cs1, cs2)


RECURRENCE_PINS = [pin_golden_worked, pin_closed_form, pin_identity_gate, pin_zero_decay,
                   pin_writes_v, pin_pure_decay, pin_rank_one, pin_tokens_compose,
                   pin_head_independence, pin_linearity, pin_scale]
PROLOGUE_PINS = [pin_conv_matches_numpy, pin_conv_bias, pin_conv_identity_taps,
                 pin_conv_state_roll, pin_unit_norm, pin_gates, pin_fused_composes]
# ----------------------------------------------------------------------------- low-rank window
#
# "GDN tuning limits on Kunlun XPU", section 三.3: the low-rank route keeps a cache of the
# most recent r rank-1 updates (not a factorisation of the state). Reading pinned here: the
# state is the sum of the last r writes of the gated delta rule, each decayed by every gate
# since it was written; slot i holds (U_i, K_i, c_i) and stands for c_i U_i K_i^T.


def lowrank_effective_state(U, K, c):
    """sum_i c_i U_i K_i^T per (sequence, head): [B,H,dv,dk]."""
    return np.einsum("bhs,bhsi,bhsj->bhij", c, U, K)


def _lowrank_filled(rng, B, H, r, dk, dv):
    U = rng.standard_normal((B, H, r, dv)) * 0.5
    K = rng.standard_normal((B, H, r, dk))
    K /= np.linalg.norm(K, axis=-1, keepdims=True)
    c = rng.uniform(0.05, 1.0, (B, H, r))
    pos = rng.integers(0, r, (B, H)).astype(np.int32)
    return U, K, c, pos


def _lowrank_empty(B, H, r, dk, dv, pos=None):
    pos = np.zeros((B, H), np.int32) if pos is None else pos
    return np.zeros((B, H, r, dv)), np.zeros((B, H, r, dk)), np.zeros((B, H, r)), pos


def pin_lowrank_long_window_is_full_rank(lib, seed=20):
    """A window at least as long as the run, from an empty start, is the full recurrence:
    the same o and the same state as oracle_gdn_decode from S0 = 0 (itself pinned above)."""
    rng = np.random.default_rng(seed)
    for r, T in ((8, 5), (8, 8), (12, 7), (3, 3)):
        q, k, v, al, be, _ = _rand_inputs(rng, 2, T, 3, 8, 8)
        pos0 = rng.integers(0, r, (2, 3)).astype(np.int32)
        U, K, c, pos = _lowrank_empty(2, 3, r, 8, 8, pos0)
        U, K, c, pos, o = oracle.gdn_lowrank_decode(q, k, v, al, be, U, K, c, pos, lib=lib)
        S_full, o_full = oracle.gdn_decode(q, k, v, al, be, np.zeros((2, 3, 8, 8)), lib=lib)
        assert np.max(np.abs(o - o_full)) <= 1e-12 * max(1.0, np.max(np.abs(o_full))), (r, T)
        S = lowrank_effective_state(U, K, c)
        assert np.max(np.abs(S - S_full)) <= 1e-12 * max(1.0, np.max(np.abs(S_full))), (r, T)
        assert np.array_equal(pos, (pos0 + T) % r), (r, T)


def pin_lowrank_orthogonal_keys(lib, seed=21):
    """Keys e_0, e_1, ... (mutually orthogonal): no write sees an earlier one, so delta_t =
    beta_t v_t, and after token t the state's column i is (alpha_{i+1}..alpha_t) beta_i v_i
    for the r most recent tokens i and exactly zero for every older one."""
    rng = np.random.default_rng(seed)
    B, H, D, r, T = 1, 2, 16, 4, 11
    q, _, v, al, be, _ = _rand_inputs(rng, B, T, H, D, D)
    k = np.zeros((B, T, H, D))
    for t in range(T):
        k[:, t, :, t] = 1.0
    U, K, c, pos = _lowrank_empty(B, H, r, D, D, np.array([[1, 3]], np.int32))
    U, K, c, pos, o = oracle.gdn_lowrank_decode(q, k, v, al, be, U, K, c, pos, scale=0.5, lib=lib)
    for h in range(H):
        for t in range(T):
            St = np.zeros((D, D))
            for i in range(max(0, t - r + 1), t + 1):
                St[:, i] = np.prod(al[0, i + 1: t + 1, h]) * be[0, i, h] * v[0, i, h]
            assert np.max(np.abs(o[0, t, h] - St @ (0.5 * q[0, t, h]))) <= 1e-13, (h, t)
        S = lowrank_effective_state(U, K, c)[0, h]
        assert np.max(np.abs(S - St)) <= 1e-14, h
        assert np.all(S[:, : T - r] == 0.0), h


def pin_lowrank_single_slot(lib, seed=22):
    """r = 1 keeps only the newest write: S_t = delta_t k_t^T with
    delta_t = beta_t (v_t - alpha_t (k_{t-1} . k_t) delta_{t-1}), and o_t = delta_t (k_t . q_t)."""
    rng = np.random.default_rng(seed)
    B, H, D, T = 1, 2, 8, 6
    q, k, v, al, be, _ = _rand_inputs(rng, B, T, H, D, D)
    U, K, c, pos = _lowrank_empty(B, H, 1, D, D)
    U, K, c, pos, o = oracle.gdn_lowrank_decode(q, k, v, al, be, U, K, c, pos, lib=lib)
    for h in range(H):
        d_prev, k_prev = np.zeros(D), np.zeros(D)
        for t in range(T):
            kt = k[0, t, h]
            d = be[0, t, h] * (v[0, t, h] - al[0, t, h] * np.dot(k_prev, kt) * d_prev)
            assert np.max(np.abs(o[0, t, h] - d * np.dot(kt, q[0, t, h]))) <= 1e-13, (h, t)
            d_prev, k_prev = d, kt
        assert np.max(np.abs(U[0, h, 0] - d_prev)) <= 1e-13 and c[0, h, 0] == 1.0


def pin_lowrank_rank_bound(lib, seed=23):
    """The state is a sum of at most r rank-1 terms: rank <= min(r, tokens seen) although the
    full recurrence on the same inputs reaches full rank."""
    rng = np.random.default_rng(seed)
    B, H, D, r, T = 1, 2, 8, 3, 12
    q, k, v, al, be, _ = _rand_inputs(rng, B, T, H, D, D)
    U, K, c, pos = _lowrank_empty(B, H, r, D, D)
    for t in range(T):
        sl = slice(t, t + 1)
        U, K, c, pos, _ = oracle.gdn_lowrank_decode(q[:, sl], k[:, sl], v[:, sl], al[:, sl],
                                                    be[:, sl], U, K, c, pos, lib=lib)
        S = lowrank_effective_state(U, K, c)
        for h in range(H):
            assert np.linalg.matrix_rank(S[0, h], tol=1e-10) == min(r, t + 1), (t, h)
    S_full, _ = oracle.gdn_decode(q, k, v, al, be, np.zeros((B, H, D, D)), lib=lib)
    assert np.linalg.matrix_rank(S_full[0, 0], tol=1e-10) == D


def lowrank_window_bruteforce(U, K, c, pos, q, k, v, al, be, scale=1.0):
    """One head by a different algorithm: the window as a queue of (decayed write, key) pairs,
    oldest first (slot pos is the oldest), each token appending its write and dropping the
    oldest, the decay applied to the stored vectors themselves. Returns (S_T, o [T, dv])."""
    r = U.shape[0]
    win = [(c[s] * U[s], K[s]) for s in ((pos + j) % r for j in range(r))]
    outs = []
    for t in range(len(al)):
        S = sum(np.outer(w, kk) for w, kk in win)
        delta = be[t] * (v[t] - al[t] * (S @ k[t]))
        win = [(al[t] * w, kk) for w, kk in win[1:]] + [(delta, k[t])]
        S = sum(np.outer(w, kk) for w, kk in win)
        outs.append(S @ (scale * q[t]))
    return S, np.array(outs)


def pin_lowrank_bruteforce(lib, seed=24):
    """A filled window (every slot in use, any next slot) against the queue brute force."""
    rng = np.random.default_rng(seed)
    B, H, D, r, T = 2, 2, 6, 3, 9
    q, k, v, al, be, _ = _rand_inputs(rng, B, T, H, D, D)
    U0, K0, c0, pos0 = _lowrank_filled(rng, B, H, r, D, D)
    U, K, c, pos, o = oracle.gdn_lowrank_decode(q, k, v, al, be, U0, K0, c0, pos0, scale=0.7,
                                                lib=lib)
    S = lowrank_effective_state(U, K, c)
    for b in range(B):
        for h in range(H):
            Sx, ox = lowrank_window_bruteforce(U0[b, h], K0[b, h], c0[b, h], pos0[b, h],
                                               q[b, :, h], k[b, :, h], v[b, :, h],
                                               al[b, :, h], be[b, :, h], scale=0.7)
            assert np.max(np.abs(S[b, h] - Sx)) <= 1e-12 * max(1.0, np.max(np.abs(Sx)))
            assert np.max(np.abs(o[b, :, h] - ox)) <= 1e-12 * max(1.0, np.max(np.abs(ox)))


def pin_lowrank_calls_resume(lib, seed=25):
    """One call of T tokens equals the same tokens split over several calls, bit for bit."""
    rng = np.random.default_rng(seed)
    B, H, D, r, T = 2, 3, 8, 4, 9
    q, k, v, al, be, _ = _rand_inputs(rng, B, T, H, D, D)
    st0 = _lowrank_filled(rng, B, H, r, D, D)
    whole = oracle.gdn_lowrank_decode(q, k, v, al, be, *st0, lib=lib)
    st, outs = st0, []
    for a, z in ((0, 4), (4, 5), (5, 9)):
        sl = slice(a, z)
        *st, o = oracle.gdn_lowrank_decode(q[:, sl], k[:, sl], v[:, sl], al[:, sl], be[:, sl],
                                           *st, lib=lib)
        outs.append(o)
    for x, y in zip(whole[:4], st):
        assert np.array_equal(x, y)
    assert np.array_equal(whole[4], np.concatenate(outs, axis=1))


def pin_lowrank_golden_worked(lib):
    """Hand-worked dyadic examples of the window (golden/gdn_lowrank_worked.json) reproduce
    exactly, token by token and in one call."""
    with open(os.path.join(GOLDEN, "gdn_lowrank_worked.json")) as f:
        doc = json.load(f)
    for case in doc["cases"]:
        toks = case["tokens"]
        T = len(toks)
        q = np.array([[t["q"] for t in toks]], dtype=float)[:, :, None, :]
        k = np.array([[t["k"] for t in toks]], dtype=float)[:, :, None, :]
        v = np.array([[t["v"] for t in toks]], dtype=float)[:, :, None, :]
        al = np.array([[t["alpha"] for t in toks]], dtype=float)[:, :, None]
        be = np.array([[t["beta"] for t in toks]], dtype=float)[:, :, None]
        U0 = np.array(case["U0"], dtype=float)[None, None]
        K0 = np.array(case["K0"], dtype=float)[None, None]
        c0 = np.array(case["c0"], dtype=float)[None, None]
        pos0 = np.array([[case["pos0"]]], dtype=np.int32)
        U, K, c, pos, o = oracle.gdn_lowrank_decode(q, k, v, al, be, U0, K0, c0, pos0, lib=lib)
        assert np.array_equal(o[0, :, 0, :], np.array([t["o"] for t in toks], dtype=float)), case["name"]
        assert np.array_equal(U[0, 0], np.array(case["U"], dtype=float)), case["name"]
        assert np.array_equal(K[0, 0], np.array(case["K"], dtype=float)), case["name"]
        assert np.array_equal(c[0, 0], np.array(case["c"], dtype=float)), case["name"]
        assert int(pos[0, 0]) == case["pos"] and o.shape == (1, T, 1, 2), case["name"]


LOWRANK_PINS = [pin_lowrank_golden_worked, pin_lowrank_long_window_is_full_rank, pin_lowrank_orthogonal_keys,
                pin_lowrank_single_slot, pin_lowrank_rank_bound, pin_lowrank_bruteforce,
                pin_lowrank_calls_resume]

ALL_PINS = RECURRENCE_PINS + PROLOGUE_PINS + LOWRANK_PINS

