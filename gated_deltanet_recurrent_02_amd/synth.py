"""Seeded synthetic inputs for the GDN decode step, shared by the tests and the benchmark.

This module only draws random numbers and shapes them into the input recipe of each workload:
it holds none of the step's arithmetic and computes no expected value. The GPU library and the
oracle both consume what it returns; neither is imported here.

Recipes (no trained weights or live activations exist for this path, so these stand in):
  * Decode-step workloads take q, k already L2-normalised and the gates as values:
      state  ~ N(0, std)            (std 0.02; "zeros" for the tiny workload)
      q, k   ~ N(0, 1), each (sequence, token, head) vector scaled to unit length in fp64
      v      ~ N(0, 1)
      beta   = logistic(z),                z ~ N(0, 1)
      alpha  = exp(-softplus(z + shift)),  z ~ N(0, 1)   (shift 2 by default; -2 for the
                                                          prompt workload, whose 4096 tokens
                                                          keep a median alpha of 0.88)
    draw order: state, q, k, v, beta-logit, alpha-logit; one PCG64 stream per workload.
  * Fused-layer workloads take raw activations:
      qkv ~ N(0, 1) bf16 [B,T,C], conv_state ~ N(0, 1) bf16 [B,C,3], conv_w ~ N(0, 0.5) fp32 [C,4],
      a_logit, b_logit ~ N(0, 1) fp32 [B,T,H], state ~ N(0, 0.02)
    draw order: qkv, conv_state, conv_w, a_logit, b_logit, state.
  * Low-rank window workloads (r slots per head) take the decode-step recipe for the tokens
    and a full window of earlier writes:
      U ~ N(0, 0.5), K ~ N(0, 1) rows scaled to unit length, pos uniform on [0, r),
      and the weight of the slot written a tokens ago is the product of a past gates drawn
      like alpha (1 for the newest slot), so older writes carry less weight;
    draw order: U, K, past gates, pos, then q, k, v, beta-logit, alpha-logit.
    `window="empty"` gives the all-zero window of a new sequence instead.
Every narrower type (bf16, fp16) is the round-to-nearest-even image of the fp32/fp64 draw
(torch's cast).
"""
from __future__ import annotations

import numpy as np
import torch

_TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}

# Named workloads: batch B, heads H, head dim D (dk = dv), tokens per call T.
WORKLOADS = {
    "decode_b1_h2_d16_t8": dict(B=1, H=2, D=16, T=8, act="f32", state_init="zeros"),
    "decode_b1_h48_d128_t1": dict(B=1, H=48, D=128, T=1, act="bf16", state_init="normal"),
    "decode_b64_h48_d128_t1": dict(B=64, H=48, D=128, T=1, act="bf16", state_init="normal"),
    "decode_b256_h48_d128_t1": dict(B=256, H=48, D=128, T=1, act="bf16", state_init="normal"),
    "decode_b256_h48_d128_t4": dict(B=256, H=48, D=128, T=4, act="bf16", state_init="normal"),
    "fused_b256_h48_d128_t4": dict(B=256, H=48, D=128, T=4, fused=True),
    # a batch of long prompts run through the recurrence in one call (prefill)
    "prefill_b4_h48_d128_t4096": dict(B=4, H=48, D=128, T=4096, act="bf16", state_init="normal",
                                      alpha_shift=-2.0, prefill=True),
    # decode on the sliding-window low-rank state: r slots per head
    "lowrank_b1_h48_d128_r16_t1": dict(B=1, H=48, D=128, T=1, act="bf16", r=16, lowrank=True),
    "lowrank_b256_h48_d128_r16_t1": dict(B=256, H=48, D=128, T=1, act="bf16", r=16, lowrank=True),
    "lowrank_b256_h48_d128_r32_t1": dict(B=256, H=48, D=128, T=1, act="bf16", r=32, lowrank=True),
    "lowrank_b256_h48_d128_r16_t4": dict(B=256, H=48, D=128, T=4, act="bf16", r=16, lowrank=True),
    "lowrank_b256_h48_d128_r32_t8": dict(B=256, H=48, D=128, T=8, act="bf16", r=32, lowrank=True),
    # speculative verify rounds of 4 tokens; the accepted prefix per sequence is drawn by
    # accepted_prefix() below
    "verify_b256_h48_d128_t4": dict(B=256, H=48, D=128, T=4, act="bf16", state_init="normal",
                                    verify=True),
}


def accepted_prefix(B: int, T: int, seed: int = 0) -> torch.Tensor:
    """Accepted draft-prefix lengths per sequence for verify rounds: uniform on [1, T] (the
    pages give no acceptance rates), int32 [B]."""
    rng = _rng(seed + 1)
    return torch.from_numpy(rng.integers(1, T + 1, B).astype(np.int32))


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _unit_rows(a: np.ndarray) -> np.ndarray:
    """Scale every last-axis vector of a float64 array to unit Euclidean length."""
    return a / np.sqrt(np.sum(a * a, axis=-1, keepdims=True))


def _cast(a: np.ndarray, dtype: str) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(_TORCH_DTYPES[dtype])


def decode_inputs(B: int, H: int, D: int, T: int, *, act: str = "bf16",
                  state_dtype: str = "f32", state_init: str = "normal",
                  state_std: float = 0.02, alpha_shift: float = 2.0, seed: int = 0) -> dict:
    """Inputs of one decode-step call, as CPU torch tensors in their device dtypes."""
    rng = _rng(seed)
    if state_init == "normal":
        s = rng.standard_normal((B, H, D, D), dtype=np.float32)
        s *= np.float32(state_std)
    elif state_init == "zeros":
        s = np.zeros((B, H, D, D), dtype=np.float32)
    else:
        raise ValueError(f"unknown state_init {state_init!r}")
    q = _unit_rows(rng.standard_normal((B, T, H, D)))
    k = _unit_rows(rng.standard_normal((B, T, H, D)))
    v = rng.standard_normal((B, T, H, D))
    zb = rng.standard_normal((B, T, H))
    za = rng.standard_normal((B, T, H)) + alpha_shift
    beta = 1.0 / (1.0 + np.exp(-zb))
    alpha = np.exp(-(np.maximum(za, 0.0) + np.log1p(np.exp(-np.abs(za)))))
    return dict(
        q=_cast(q.astype(np.float32), act), k=_cast(k.astype(np.float32), act),
        v=_cast(v.astype(np.float32), act),
        alpha=_cast(alpha.astype(np.float32), "f32"), beta=_cast(beta.astype(np.float32), "f32"),
        state=_cast(s, state_dtype),
        B=B, H=H, D=D, T=T, act=act, state_dtype=state_dtype,
    )


def fused_inputs(B: int, H: int, D: int, T: int, *, state_dtype: str = "f32",
                 state_std: float = 0.02, conv_w_std: float = 0.5, with_bias: bool = False,
                 seed: int = 0) -> dict:
    """Inputs of one fused-layer call (conv + gates + T steps), CPU torch tensors."""
    rng = _rng(seed)
    C = 3 * H * D
    qkv = rng.standard_normal((B, T, C), dtype=np.float32)
    cs = rng.standard_normal((B, C, 3), dtype=np.float32)
    w = rng.standard_normal((C, 4), dtype=np.float32) * np.float32(conv_w_std)
    a = rng.standard_normal((B, T, H), dtype=np.float32)
    b = rng.standard_normal((B, T, H), dtype=np.float32)
    s = rng.standard_normal((B, H, D, D), dtype=np.float32)
    s *= np.float32(state_std)
    bias = rng.standard_normal((C,), dtype=np.float32) * np.float32(0.1) if with_bias else None
    return dict(
        qkv=_cast(qkv, "bf16"), conv_state=_cast(cs, "bf16"), conv_w=_cast(w, "f32"),
        conv_b=None if bias is None else _cast(bias, "f32"),
        a_logit=_cast(a, "f32"), b_logit=_cast(b, "f32"), state=_cast(s, state_dtype),
        B=B, H=H, D=D, T=T, state_dtype=state_dtype,
    )


def lowrank_inputs(B: int, H: int, D: int, T: int, r: int, *, act: str = "bf16",
                   state_dtype: str = "f32", window: str = "filled", u_std: float = 0.5,
                   alpha_shift: float = 2.0, seed: int = 0) -> dict:
    """Inputs of one low-rank window call, as CPU torch tensors: the decode-step token recipe
    plus a window state U [B,H,r,D], K [B,H,r,D] (state dtype), c fp32 [B,H,r], pos int32 [B,H]."""
    rng = _rng(seed)
    if window == "filled":
        U = rng.standard_normal((B, H, r, D)) * u_std
        K = _unit_rows(rng.standard_normal((B, H, r, D)))
        zp = rng.standard_normal((B, H, r)) + alpha_shift
        past = np.exp(-(np.maximum(zp, 0.0) + np.log1p(np.exp(-np.abs(zp)))))
        pos = rng.integers(0, r, (B, H)).astype(np.int32)
        by_age = np.concatenate([np.ones((B, H, 1)), np.cumprod(past, axis=-1)[..., :-1]], axis=-1)
        age = (pos[..., None] - 1 - np.arange(r)) % r          # 0 = the newest slot
        c = np.take_along_axis(by_age, age, axis=-1)
    elif window == "empty":
        U = np.zeros((B, H, r, D)); K = np.zeros((B, H, r, D)); c = np.zeros((B, H, r))
        pos = np.zeros((B, H), np.int32)
    else:
        raise ValueError(f"unknown window {window!r}")
    q = _unit_rows(rng.standard_normal((B, T, H, D)))
    k = _unit_rows(rng.standard_normal((B, T, H, D)))
    v = rng.standard_normal((B, T, H, D))
    zb = rng.standard_normal((B, T, H))
    za = rng.standard_normal((B, T, H)) + alpha_shift
    beta = 1.0 / (1.0 + np.exp(-zb))
    alpha = np.exp(-(np.maximum(za, 0.0) + np.log1p(np.exp(-np.abs(za)))))
    return dict(
        q=_cast(q.astype(np.float32), act), k=_cast(k.astype(np.float32), act),
        v=_cast(v.astype(np.float32), act),
        alpha=_cast(alpha.astype(np.float32), "f32"), beta=_cast(beta.astype(np.float32), "f32"),
        U=_cast(U.astype(np.float32), state_dtype), K=_cast(K.astype(np.float32), state_dtype),
        c=_cast(c.astype(np.float32), "f32"), pos=torch.from_numpy(np.ascontiguousarray(pos)),
        B=B, H=H, D=D, T=T, r=r, act=act, state_dtype=state_dtype,
    )


def workload_inputs(name: str, *, seed: int = 0, **overrides) -> dict:
    """Inputs of a named workload (see WORKLOADS); keyword overrides replace recipe fields."""
    spec = dict(WORKLOADS[name])
    fused = spec.pop("fused", False)
    spec.pop("verify", False)
    spec.pop("prefill", False)
    lowrank = spec.pop("lowrank", False)
    spec.update(overrides)
    if lowrank:
        spec.pop("state_init", None)
        return lowrank_inputs(seed=seed, **spec)
    if fused:
        return fused_inputs(seed=seed, **spec)
    return decode_inputs(seed=seed, **spec)
