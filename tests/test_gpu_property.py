"""Property tests on the GPU: random shapes, dtypes, token counts and seeds, drawn by
hypothesis (derandomized, so every run draws the same cases), each compared with the fp64
oracle at the parity bars. Covers gdn_decode_step and gdn_lowrank_decode_step."""
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from gated_deltanet_recurrent_02_amd import synth
from parity import (check_lowrank, check_o, check_state, f64, gpu_decode, gpu_lowrank,
                    oracle_decode, oracle_lowrank)

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
SETTINGS = settings(max_examples=40, deadline=None, derandomize=True, database=None,
                    suppress_health_check=[HealthCheck.too_slow])


@SETTINGS
@given(B=st.integers(1, 8), H=st.integers(1, 6), T=st.integers(1, 9),
       D=st.sampled_from([16, 32, 64, 128]), act=st.sampled_from(["f32", "bf16", "f16"]),
       sdt=st.sampled_from(["f32", "bf16", "f16"]), shift=st.sampled_from([2.0, -2.0]),
       scale=st.sampled_from([1.0, 0.5]), seed=st.integers(0, 2 ** 16))
def test_decode_step_random_cases(B, H, T, D, act, sdt, shift, scale, seed):
    print(f"[case] decode B={B} H={H} T={T} D={D} act={act} state={sdt} seed={seed}", flush=True)
    x = synth.decode_inputs(B, H, D, T, act=act, state_dtype=sdt, alpha_shift=shift,
                            state_std=0.3, seed=seed)
    S, o = gpu_decode(x, scale=scale)
    S_ref, o_ref = oracle_decode(x, scale=scale)
    check_state(f64(S), S_ref, DT[sdt])
    check_o(f64(o), o_ref, DT[act])


@SETTINGS
@given(B=st.integers(1, 4), H=st.integers(1, 6), T=st.integers(1, 24),
       D=st.sampled_from([16, 32, 64, 128]), r=st.sampled_from([8, 16, 32]),
       act=st.sampled_from(["f32", "bf16", "f16"]), sdt=st.sampled_from(["f32", "bf16"]),
       window=st.sampled_from(["filled", "empty"]), seed=st.integers(0, 2 ** 16))
def test_lowrank_random_cases(B, H, T, D, r, act, sdt, window, seed):
    print(f"[case] lowrank B={B} H={H} T={T} D={D} r={r} act={act} state={sdt} {window} "
          f"seed={seed}", flush=True)
    x = synth.lowrank_inputs(B, H, D, T, r, act=act, state_dtype=sdt, window=window, seed=seed)
    g, o = gpu_lowrank(x)
    check_lowrank(g, o, oracle_lowrank(x), DT[act], DT[sdt])
