"""Both step functions are graph-capturable (no host sync, allocation or memset inside):
capture a call in a HIP graph via torch, replay it several times with eager work and
synchronisation in between, and check every replay against the same call run eagerly."""
import pytest
import torch

import gated_deltanet_recurrent_02_amd as gdn
from gated_deltanet_recurrent_02_amd import synth
from parity import to_dev

pytestmark = pytest.mark.gpu


def _announce(msg):
    print(f"[case] {msg}", flush=True)


@pytest.mark.parametrize("T,sdt", [(1, "f32"), (4, "bf16")])
def test_decode_step_graph_replays_match_eager(T, sdt):
    _announce(f"graph decode T={T} state={sdt}")
    x = to_dev(synth.decode_inputs(8, 48, 128, T, state_dtype=sdt, seed=30 + T))
    S0 = x["state"].clone()
    # eager reference for 3 consecutive calls
    ref_S, ref_o = S0.clone(), []
    for _ in range(3):
        ref_o.append(gdn.decode_step(x["q"], x["k"], x["v"], x["alpha"], x["beta"], ref_S).clone())
    torch.cuda.synchronize()
    S = S0.clone()
    o = torch.empty_like(x["v"])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm the binding on the capture stream
        gdn.decode_step(x["q"], x["k"], x["v"], x["alpha"], x["beta"], S.clone(), o=o)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gdn.decode_step(x["q"], x["k"], x["v"], x["alpha"], x["beta"], S, o=o)
    S.copy_(S0)
    for i in range(3):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), ref_o[i].view(torch.int16)), f"o of replay {i}"
        _ = (S.float().sum() if sdt == "f32" else S.float().abs().max())  # eager work between
    assert torch.equal(S.view(torch.int16), ref_S.view(torch.int16))


@pytest.mark.parametrize("sdt", ["f32", "bf16"])
def test_decode_verify_graph_replays_match_eager(sdt):
    # A verify call that commits the previous round's accepted prefix and drafts 4 new tokens
    # (a bf16 state: the chunk-form kernel), captured once and replayed on the evolving state.
    _announce(f"graph verify T=4 state={sdt}")
    x1 = to_dev(synth.decode_inputs(8, 48, 128, 4, state_dtype=sdt, alpha_shift=-1.0, seed=36))
    x2 = to_dev(synth.decode_inputs(8, 48, 128, 4, state_dtype=sdt, alpha_shift=-1.0, seed=37))
    tok = lambda x: (x["q"], x["k"], x["v"], x["alpha"], x["beta"])
    S0 = x1["state"].clone()
    _, d1 = gdn.decode_verify(*tok(x1), S0.clone())
    n = torch.tensor([0, 1, 2, 3, 4, 4, 2, 1], dtype=torch.int32, device="cuda")
    prev = (n, x1["k"], x1["alpha"], d1)
    ref_S, ref = S0.clone(), []
    for _ in range(3):
        o_r, d_r = gdn.decode_verify(*tok(x2), ref_S, prev=prev)
        ref.append((o_r.clone(), d_r.clone()))
    torch.cuda.synchronize()
    S = S0.clone()
    o = torch.empty_like(x2["v"])
    dk = torch.empty(o.shape, dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm the binding on the capture stream
        gdn.decode_verify(*tok(x2), S.clone(), prev=prev, o=o, dk_out=dk)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gdn.decode_verify(*tok(x2), S, prev=prev, o=o, dk_out=dk)
    S.copy_(S0)
    for i in range(3):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), ref[i][0].view(torch.int16)), f"o of replay {i}"
        assert torch.equal(dk, ref[i][1]), f"dk of replay {i}"
        _ = S.float().abs().max()  # eager work between replays
    assert torch.equal(S.view(torch.int16), ref_S.view(torch.int16))


def test_conv_gate_decode_graph_replays_match_eager():
    _announce("graph fused T=4")
    x = to_dev(synth.fused_inputs(8, 48, 128, 4, seed=33))
    S0, cs0 = x["state"].clone(), x["conv_state"].clone()
    ref_S, ref_cs, ref_o = S0.clone(), cs0.clone(), []
    for _ in range(3):
        ref_o.append(gdn.conv_gate_decode(x["qkv"], ref_cs, x["conv_w"], None, x["a_logit"],
                                          x["b_logit"], ref_S).clone())
    torch.cuda.synchronize()
    S, cs = S0.clone(), cs0.clone()
    o = torch.empty((8, 4, 48, 128), dtype=torch.bfloat16, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gdn.conv_gate_decode(x["qkv"], cs, x["conv_w"], None, x["a_logit"], x["b_logit"], S, o=o)
    S.copy_(S0)
    cs.copy_(cs0)
    for i in range(3):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), ref_o[i].view(torch.int16)), f"o of replay {i}"
        _ = cs.float().sum()
    assert torch.equal(S, ref_S) and torch.equal(cs.view(torch.int16), ref_cs.view(torch.int16))


def test_prefill_graph_replays_match_eager():
    # Both prefill kernels in one captured graph with a workspace allocated beforehand.
    _announce("graph prefill B=2 H=8 D=128 T=100")
    x = to_dev(synth.decode_inputs(2, 8, 128, 100, alpha_shift=-2.0, seed=34))
    S0 = x["state"].clone()
    ws = gdn.prefill_workspace(x["q"], x["v"])
    ref_S, ref_o = S0.clone(), []
    for _ in range(3):
        ref_o.append(gdn.prefill(x["q"], x["k"], x["v"], x["alpha"], x["beta"], ref_S, workspace=ws).clone())
    torch.cuda.synchronize()
    S = S0.clone()
    o = torch.empty_like(x["v"])
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gdn.prefill(x["q"], x["k"], x["v"], x["alpha"], x["beta"], S, o=o, workspace=ws)
    S.copy_(S0)
    for i in range(3):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), ref_o[i].view(torch.int16)), f"o of replay {i}"
        _ = S.float().abs().max()  # eager work between replays
    assert torch.equal(S, ref_S)
