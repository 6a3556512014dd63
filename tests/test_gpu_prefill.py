"""gdn_prefill (the chunked form of T tokens) on the GPU against the fp64 oracle.

The oracle is the plain recurrence token by token (oracle_gdn_decode); the chunked form must
reach the same state and outputs within the floating-point bars of parity.py. Small shapes are
compared on every head, with ragged last chunks (T not a multiple of 16) and several chunks
(bf16 activations take the chunks in pairs: even and odd chunk counts, a ragged second chunk
of a pair and a ragged lone last chunk are all covered); the prompt workload (B=4, H=48, D=128,
T=4096) on every head.
"""
import numpy as np
import pytest
import torch

import gated_deltanet_recurrent_02_amd as gdn
import oracle
from gated_deltanet_recurrent_02_amd import synth
from parity import check_o, check_state, f64, oracle_decode, oracle_decode_all, to_dev

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _announce(msg):
    print(f"[case] {msg}", flush=True)


def gpu_prefill(x, scale=1.0, workspace=None):
    g = to_dev(x)
    o = gdn.prefill(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["state"], scale=scale,
                    workspace=workspace)
    torch.cuda.synchronize()
    return g["state"], o


@pytest.mark.parametrize("D", [16, 32, 64, 128])
@pytest.mark.parametrize("act", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("B,H,T", [(2, 3, 1), (1, 2, 16), (2, 2, 20), (3, 2, 37), (2, 2, 60),
                                   (1, 3, 100)])
def test_small_shapes_full_compare(D, act, B, H, T):
    _announce(f"prefill B={B} H={H} D={D} T={T} act={act} state=f32")
    x = synth.decode_inputs(B, H, D, T, act=act, alpha_shift=-2.0, state_std=0.3, seed=D + T)
    S, o = gpu_prefill(x, scale=0.7)
    S_ref, o_ref = oracle_decode(x, scale=0.7)
    check_state(f64(S), S_ref, torch.float32)
    check_o(f64(o), o_ref, DT[act])


@pytest.mark.parametrize("sdt", ["bf16", "f16"])
@pytest.mark.parametrize("T", [5, 48, 77])
def test_16bit_state(sdt, T):
    _announce(f"prefill B=2 H=4 D=128 T={T} act=bf16 state={sdt}")
    x = synth.decode_inputs(2, 4, 128, T, act="bf16", state_dtype=sdt, alpha_shift=-2.0,
                            state_std=0.3, seed=T)
    S, o = gpu_prefill(x)
    S_ref, o_ref = oracle_decode(x)
    check_state(f64(S), S_ref, DT[sdt])
    check_o(f64(o), o_ref, torch.bfloat16)


@pytest.mark.parametrize("sdt", ["f32", "bf16"])
def test_prompt_workload_all_heads(sdt):
    # All 192 heads of the prompt workload over all 4096 tokens against the oracle (run on a
    # thread pool).
    name = "prefill_b4_h48_d128_t4096"
    _announce(f"{name} state={sdt}")
    x = synth.workload_inputs(name, state_dtype=sdt)
    S, o = gpu_prefill(x)
    S_ref, o_ref = oracle_decode_all(x)
    check_state(f64(S), S_ref, DT[sdt])
    check_o(f64(o), o_ref, torch.bfloat16)


def test_agrees_with_decode_step():
    # The same call through the token-by-token kernel: both within the bars of the oracle, and
    # the two fp32 states within the fp32 bar of each other.
    _announce("prefill vs decode_step B=2 H=6 D=128 T=300")
    x = synth.decode_inputs(2, 6, 128, 300, act="bf16", alpha_shift=-2.0, seed=11)
    S_p, o_p = gpu_prefill(x)
    g = to_dev(x)
    o_d = gdn.decode_step(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["state"])
    torch.cuda.synchronize()
    S_ref, o_ref = oracle_decode(x)
    for S, o in ((S_p, o_p), (g["state"], o_d)):
        check_state(f64(S), S_ref, torch.float32)
        check_o(f64(o), o_ref, torch.bfloat16)
    check_state(f64(S_p), f64(g["state"]), torch.float32)


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_gate_edge_values(act):
    # alpha = 0 wipes the state at that token (the products of alphas carry the exact zero);
    # beta = 0 leaves a token without a write; a zero key writes nothing.
    _announce(f"prefill gate edge values act={act}")
    x = synth.decode_inputs(2, 3, 64, 50, act=act, alpha_shift=-2.0, state_std=0.3, seed=3)
    x["alpha"][0, 7, :] = 0.0
    x["alpha"][1, 16, 1] = 0.0      # first token of the second chunk
    x["alpha"][1, 31, 2] = 0.0      # last token of the second chunk
    x["beta"][0, 20:24, :] = 0.0
    x["k"][1, 40, 0] = 0.0
    x["alpha"][0, 45:, 2] = 1.0
    S, o = gpu_prefill(x, scale=0.5)
    S_ref, o_ref = oracle_decode(x, scale=0.5)
    check_state(f64(S), S_ref, torch.float32)
    check_o(f64(o), o_ref, DT[act])


def test_workspace_contents_do_not_matter():
    _announce("prefill stale workspace")
    x = synth.decode_inputs(2, 4, 32, 45, act="bf16", seed=4)
    ws = gdn.prefill_workspace(x["q"].cuda(), x["v"].cuda())
    ws.view(torch.float32).fill_(float("nan"))
    S1, o1 = gpu_prefill(x, workspace=ws)
    S2, o2 = gpu_prefill(x)
    assert torch.equal(S1, S2) and torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_deterministic():
    _announce("prefill determinism")
    x = synth.decode_inputs(4, 8, 128, 70, act="bf16", seed=6)
    S1, o1 = gpu_prefill(x)
    S2, o2 = gpu_prefill(x)
    assert torch.equal(S1, S2) and torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_empty_calls_leave_state_unchanged():
    _announce("prefill empty calls")
    for B, T in ((0, 5), (2, 0)):
        x = synth.decode_inputs(max(B, 1), 2, 16, max(T, 1), act="f32", seed=7)
        st = x["state"].cuda()[:B] if B == 0 else x["state"].cuda()
        q = x["q"].cuda()[:B, :T].contiguous()
        v = x["v"].cuda()[:B, :T].contiguous()
        a = x["alpha"].cuda()[:B, :T].contiguous()
        before = st.clone()
        o = gdn.prefill(q, q, v, a, a.clone(), st)
        torch.cuda.synchronize()
        assert o.numel() == 0 and torch.equal(st, before)


def test_split_calls_continue_the_state():
    # Two calls of 40 and 33 tokens equal one call of 73 (the state carries everything).
    _announce("prefill split calls")
    x = synth.decode_inputs(2, 3, 128, 73, act="f32", alpha_shift=-2.0, seed=8)
    g = to_dev(x)
    o1 = gdn.prefill(*(g[n][:, :40].contiguous() for n in ("q", "k", "v", "alpha", "beta")), g["state"])
    o2 = gdn.prefill(*(g[n][:, 40:].contiguous() for n in ("q", "k", "v", "alpha", "beta")), g["state"])
    torch.cuda.synchronize()
    S_ref, o_ref = oracle_decode(x)
    check_state(f64(g["state"]), S_ref, torch.float32)
    check_o(np.concatenate([f64(o1), f64(o2)], axis=1), o_ref, torch.float32)


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_decay_fold_paths(act):
    # The kernel keeps S / c in registers with c the running product of chunk decays and folds
    # c into the state when it leaves [2^-64, 2^64]: alpha > 1 (c grows past 2^64 within a few
    # chunks), alpha < 0 (c changes sign: folded every chunk), tiny alphas (c underflows), and
    # exact zeros mid-chunk, each on its own head.
    _announce(f"prefill decay fold paths act={act}")
    x = synth.decode_inputs(1, 4, 128, 100, act=act, state_std=0.3, seed=9)
    x["alpha"][0, :, 0] = 1.7
    x["alpha"][0, :, 1] = -0.9
    x["alpha"][0, :, 2] = 1e-3
    x["alpha"][0, 5::16, 3] = 0.0
    S, o = gpu_prefill(x, scale=0.25)
    S_ref, o_ref = oracle_decode(x, scale=0.25)
    check_state(f64(S), S_ref, torch.float32)
    check_o(f64(o), o_ref, DT[act])


def test_offsets_beyond_2_31_elements():
    # B=16 x T=32768 x H=48 x D=128 = 3.2e9 elements per activation tensor (6.4 GB of bf16 each),
    # so token offsets pass 2^31; 2048 chunks per head. Drawn on the device from a seeded
    # generator; sampled heads (including the last sequence's last head) are read back and
    # compared with the oracle over all 32768 tokens.
    B, T, H, D = 16, 32768, 48, 128
    _announce(f"prefill B={B} T={T} H={H} D={D} (3.2e9-element activations)")
    gen = torch.Generator(device="cuda").manual_seed(41)

    def unit(shape):
        x = torch.randn(shape, device="cuda", generator=gen)
        x /= x.norm(dim=-1, keepdim=True)
        return x.bfloat16()

    q, k = unit((B, T, H, D)), unit((B, T, H, D))
    v = torch.randn((B, T, H, D), device="cuda", generator=gen).bfloat16()
    alpha = torch.rand((B, T, H), device="cuda", generator=gen).mul_(0.3).add_(0.7)
    beta = torch.rand((B, T, H), device="cuda", generator=gen)
    state = torch.randn((B, H, D, D), device="cuda", generator=gen).mul_(0.3)
    heads = [(0, 0), (B // 2, 7), (B - 1, H - 1)]
    bi, hi = (torch.as_tensor(a) for a in np.asarray(heads).T)
    sel = lambda t: f64(t[bi.cuda(), :, hi.cuda()])          # [n, T, ...]
    qs, ks, vs, als, bes = (sel(t) for t in (q, k, v, alpha, beta))
    S0 = f64(state[bi.cuda(), hi.cuda()])
    o = gdn.prefill(q, k, v, alpha, beta, state)
    torch.cuda.synchronize()
    S1, o_s = f64(state[bi.cuda(), hi.cuda()]), sel(o)
    del q, k, v, o
    S_ref, o_ref = oracle.gdn_decode(qs[:, :, None], ks[:, :, None], vs[:, :, None],
                                     als[:, :, None], bes[:, :, None], S0[:, None])
    for n, (b, h) in enumerate(heads):
        check_state(S1[n][None], S_ref[n], torch.float32, what=f"state of head ({b}, {h})")
        check_o(o_s[n][None], o_ref[n, :, 0][None], torch.bfloat16)


def test_nan_stays_in_its_head():
    # A NaN in one head's initial state, and a NaN in another head's last token, reach only
    # those heads. The state NaN stays in its row. The last-token NaN does not reach the earlier
    # chunks of its head; within its own 16-token chunk the matrix products multiply it by
    # the structural zeros of T diag(beta) and P (0 * NaN = NaN), so the earlier outputs of that
    # chunk are not asserted (a documented property of the chunked form).
    _announce("prefill NaN isolation")
    x = synth.decode_inputs(3, 5, 64, 37, act="f32", seed=12)
    x["state"][1, 2, 17, 5] = float("nan")
    x["v"][2, 36, 4, 9] = float("nan")
    S, o = gpu_prefill(x)
    S, o = S.cpu(), o.cpu()
    bad_s = torch.isnan(S).any(dim=(2, 3))
    bad_o = torch.isnan(o).any(dim=(1, 3))
    expect = torch.zeros(3, 5, dtype=torch.bool)
    expect[1, 2] = True
    expect[2, 4] = True
    assert torch.equal(bad_s, expect) and torch.equal(bad_o, expect)
    assert torch.isnan(S[1, 2]).any(dim=1).nonzero().flatten().tolist() == [17]
    assert torch.isnan(o[1, :, 2]).any(dim=0).nonzero().flatten().tolist() == [17]
    assert not torch.isnan(o[2, :32, 4]).any()
    assert torch.isnan(o[2, 36, 4, 9])


@pytest.mark.parametrize("tok", [5, 20])
def test_nan_in_a_chunk_pair_stays_in_its_row(tok):
    # bf16 activations (chunks taken in pairs): a NaN in one v entry (row 9) at token 5 (first
    # chunk of the first pair) or 20 (second chunk) reaches row 9 of the state and of every
    # later output of that head, and nothing else: the other rows, heads and sequences stay
    # finite, and so do the outputs of the chunks before the NaN's own chunk.
    _announce(f"prefill bf16 NaN at token {tok}")
    x = synth.decode_inputs(2, 3, 128, 64, act="bf16", alpha_shift=-2.0, seed=13)
    x["v"][1, tok, 2, 9] = float("nan")
    S, o = gpu_prefill(x)
    S, o = S.cpu().float(), o.cpu().float()
    assert torch.isnan(S[1, 2]).any(dim=1).nonzero().flatten().tolist() == [9]
    mask = torch.ones(2, 3, dtype=torch.bool)
    mask[1, 2] = False
    assert not torch.isnan(S[mask]).any() and not torch.isnan(o.permute(0, 2, 1, 3)[mask]).any()
    head = o[1, :, 2]                                   # [T, D]
    first = 16 * (tok // 16)                            # the NaN's chunk starts here
    assert not torch.isnan(head[:first]).any()
    assert torch.isnan(head[max(tok, first + 16):, 9]).all()
    others = torch.ones(128, dtype=torch.bool)
    others[9] = False
    assert not torch.isnan(head[:, others]).any()


@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("D,T", [(128, 512), (128, 530), (64, 785), (128, 1040), (32, 2063)])
def test_long_prompts(act, D, T):
    # Long prompts on small batches: 32 chunks, 34 with a ragged last chunk, 50, 65 (odd count)
    # and 129 (odd count, ragged last chunk). Decays below one on some heads, exact zeros every
    # 29 tokens on one head and sign changes on another, so the scaled state folds many times.
    _announce(f"prefill long B=2 H=3 D={D} T={T} act={act}")
    x = synth.decode_inputs(2, 3, D, T, act=act, alpha_shift=-1.0, state_std=0.3, seed=T)
    x["alpha"][0, 7::29, 1] = 0.0
    x["alpha"][1, :, 2] = -0.97
    S, o = gpu_prefill(x, scale=0.6)
    S_ref, o_ref = oracle_decode(x, scale=0.6)
    check_state(f64(S), S_ref, torch.float32)
    check_o(f64(o), o_ref, DT[act])


def test_calls_back_to_back_on_a_side_stream():
    # Three calls continuing one state, queued on a non-default stream with no synchronisation
    # between them and sharing one workspace: each call's prep kernel overwrites the records the
    # previous call's state kernel read, so the stream order must hold.
    _announce("prefill back-to-back calls on a side stream")
    T = 3 * 600
    x = synth.decode_inputs(2, 4, 128, T, act="bf16", alpha_shift=-1.0, state_std=0.3, seed=77)
    g = to_dev(x)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    with torch.cuda.stream(side):
        ws = gdn.prefill_workspace(g["q"][:, :600], g["v"][:, :600])
        for i in range(3):
            part = [g[n][:, 600 * i:600 * (i + 1)].contiguous() for n in ("q", "k", "v", "alpha", "beta")]
            outs.append(gdn.prefill(*part, g["state"], workspace=ws))
    torch.cuda.synchronize()
    S_ref, o_ref = oracle_decode(x)
    check_state(f64(g["state"]), S_ref, torch.float32)
    check_o(np.concatenate([f64(o) for o in outs], axis=1), o_ref, torch.bfloat16)


def test_graph_capture_of_a_long_prompt():
    # A captured call replayed three times: each replay restarts from the same initial state
    # (copied in by the graph) and is compared with the oracle, with an eager call on other
    # buffers and the same workspace between the replays.
    _announce("prefill graph capture, long prompt")
    x = synth.decode_inputs(1, 4, 128, 700, act="bf16", alpha_shift=-1.0, state_std=0.3, seed=78)
    g = to_dev(x)
    S0 = g["state"].clone()
    ws = gdn.prefill_workspace(g["q"], g["v"])
    o = torch.empty_like(g["v"])
    S_ref, o_ref = oracle_decode(x)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        g["state"].copy_(S0)
        gdn.prefill(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["state"], o=o, workspace=ws)
    for rep in range(3):
        g["state"].fill_(float("nan"))
        o.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        check_state(f64(g["state"]), S_ref, torch.float32, what=f"state after replay {rep}")
        check_o(f64(o), o_ref, torch.bfloat16)
        y = to_dev(x)
        gdn.prefill(y["q"], y["k"], y["v"], y["alpha"], y["beta"], y["state"], workspace=ws)
        torch.cuda.synchronize()
        check_state(f64(y["state"]), S_ref, torch.float32, what=f"eager state after replay {rep}")


@pytest.mark.parametrize("sdt", ["f32", "bf16"])
@pytest.mark.parametrize("T", [1, 7, 15])
def test_short_prompts_take_the_decode_kernel(sdt, T):
    # Fewer than 16 tokens run on gdn_decode_step's kernel: bit-identical results, and the
    # workspace (filled with NaN) is left as it was.
    _announce(f"prefill short prompt T={T} state={sdt}")
    x = synth.decode_inputs(3, 5, 128, T, act="bf16", state_dtype=sdt, alpha_shift=-1.0,
                            state_std=0.3, seed=90 + T)
    g, d = to_dev(x), to_dev(x)
    ws = gdn.prefill_workspace(g["q"], g["v"])
    ws.view(torch.uint8).fill_(0xFF)
    before = ws.clone()
    tok = ("q", "k", "v", "alpha", "beta")
    o1 = gdn.prefill(*(g[n] for n in tok), g["state"], workspace=ws)
    o2 = gdn.decode_step(*(d[n] for n in tok), d["state"])
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(g["state"].view(torch.uint8), d["state"].view(torch.uint8))
    assert torch.equal(ws, before)
    S_ref, o_ref = oracle_decode(x)
    check_state(f64(g["state"]), S_ref, DT[sdt])
    check_o(f64(o1), o_ref, torch.bfloat16)
