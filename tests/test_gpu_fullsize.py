"""Every workload the benchmark times, at its exact shape and launch configuration, compared
with the fp64 oracle on every head (the oracle runs on a host thread pool).

Covered here: the four-token decode, the fused layer path (all 256 sequences), the verify
rounds with an accepted-prefix commit, and the three sliding-window low-rank workloads. The
one-token decode workloads and the prompt workload are compared on every head in
test_gpu_decode.py and test_gpu_prefill.py.
"""
import numpy as np
import pytest
import torch

import gated_deltanet_recurrent_02_amd as gdn
import oracle
from gated_deltanet_recurrent_02_amd import synth
from parity import (as_stored, stored_state_slack, check_lowrank, check_o, check_state, f64, gpu_decode, gpu_lowrank,
                    oracle_decode_all, oracle_lowrank, oracle_prefix_all, per_sequence, to_dev)

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _announce(msg):
    print(f"[case] {msg}", flush=True)


@pytest.mark.parametrize("sdt", ["f32", "bf16", "f16"])
def test_decode_t4_workload_all_heads(sdt):
    name = "decode_b256_h48_d128_t4"
    _announce(f"{name} state={sdt} (all 12288 heads)")
    x = synth.workload_inputs(name, state_dtype=sdt)
    S, o = gpu_decode(x)
    S_ref, o_ref = oracle_decode_all(x)
    check_state(f64(S), S_ref, DT[sdt])
    check_o(f64(o), o_ref, torch.bfloat16)


@pytest.mark.parametrize("sdt", ["f32", "bf16", "f16"])
def test_fused_workload_all_sequences(sdt):
    name = "fused_b256_h48_d128_t4"
    _announce(f"{name} state={sdt} (all 256 sequences)")
    x = synth.workload_inputs(name, state_dtype=sdt)
    g = to_dev(x)
    o = gdn.conv_gate_decode(g["qkv"], g["conv_state"], g["conv_w"], None, g["a_logit"],
                             g["b_logit"], g["state"])
    torch.cuda.synchronize()
    H, D = x["H"], x["D"]
    w = f64(x["conv_w"])

    def one(b):
        return oracle.gdn_conv_gate_decode(
            f64(x["qkv"][b:b + 1]), f64(x["conv_state"][b:b + 1]), w, None,
            f64(x["a_logit"][b:b + 1]), f64(x["b_logit"][b:b + 1]), f64(x["state"][b:b + 1]),
            H=H, dk=D, dv=D)

    parts = per_sequence(one, x["B"])
    S_ref = np.concatenate([p[0] for p in parts])
    o_ref = np.concatenate([p[1] for p in parts])
    cs_ref = np.concatenate([p[2] for p in parts])
    del parts
    assert np.array_equal(f64(g["conv_state"]), cs_ref), "conv state differs"
    check_state(f64(g["state"]), S_ref, DT[sdt])
    check_o(f64(o), o_ref, torch.bfloat16)


@pytest.mark.parametrize("sdt", ["f32", "bf16"])
def test_verify_workload_rounds_all_heads(sdt):
    # The benchmark's verify round at its shape: B=256, H=48, D=128, T=4 drafted tokens per
    # round, the previous round's accepted prefix (synth.accepted_prefix) committed first.
    # Round 1 starts from the workload's state; round 2 commits round 1's prefix and verifies
    # new tokens; a final commit-only call (T = 0) commits round 2's prefix. Every head's o of
    # both rounds and both committed states are compared with compositions of the oracle.
    name = "verify_b256_h48_d128_t4"
    _announce(f"{name} state={sdt} (two rounds + commit, all 12288 heads)")
    x1 = synth.workload_inputs(name, state_dtype=sdt)
    x2 = synth.workload_inputs(name, state_dtype=sdt, seed=1)
    B, T = x1["B"], x1["T"]
    n1 = synth.accepted_prefix(B, T)
    n2 = synth.accepted_prefix(B, T, seed=5)
    tok = ("q", "k", "v", "alpha", "beta")
    g1, g2 = to_dev(x1), to_dev(x2)
    state = g1["state"]
    o1, d1 = gdn.decode_verify(*(g1[n] for n in tok), state)
    o2, d2 = gdn.decode_verify(*(g2[n] for n in tok), state,
                               prev=(n1.cuda(), g1["k"], g1["alpha"], d1))
    torch.cuda.synchronize()
    S_c1 = f64(state)
    empty = tuple(g2[n][:, :0].contiguous() for n in tok)
    gdn.decode_verify(*empty, state, prev=(n2.cuda(), g2["k"], g2["alpha"], d2))
    torch.cuda.synchronize()
    S_c2 = f64(state)
    o1, o2 = f64(o1), f64(o2)
    del g1, g2, d1, d2, state

    _, o1_ref = oracle_decode_all(x1)
    check_o(o1, o1_ref, torch.bfloat16)
    del o1_ref
    S1c = oracle_prefix_all(x1, n1.tolist())
    check_state(S_c1, S1c, DT[sdt], what="committed state after round 1's prefix")
    # round 2 runs from the committed state as stored
    x2s = dict(x2, state=torch.from_numpy(as_stored(S1c, DT[sdt])))
    _, o2_ref = oracle_decode_all(x2s)
    check_o(o2, o2_ref, torch.bfloat16,
            extra=stored_state_slack(x2s["state"].numpy(), f64(x2["q"]), DT[sdt]))
    del o2_ref
    S2c = oracle_prefix_all(x2s, n2.tolist())
    check_state(S_c2, S2c, DT[sdt], what="committed state after round 2's prefix")


@pytest.mark.parametrize("name", ["lowrank_b256_h48_d128_r16_t1", "lowrank_b256_h48_d128_r32_t1",
                                  "lowrank_b256_h48_d128_r16_t4", "lowrank_b256_h48_d128_r32_t8"])
@pytest.mark.parametrize("sdt", ["f32", "bf16"])
def test_lowrank_workloads_all_heads(name, sdt):
    _announce(f"{name} state={sdt} (all 12288 heads)")
    x = synth.workload_inputs(name, state_dtype=sdt)
    g, o = gpu_lowrank(x)
    check_lowrank(g, o, oracle_lowrank(x), torch.bfloat16, DT[sdt])
