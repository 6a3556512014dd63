"""gdn_lowrank_decode_step (the sliding-window low-rank state) on the GPU against the fp64
oracle, plus the cross-check with the full recurrence and edge cases.

Small shapes are compared over every head and slot: every head size, every window length,
the dtype combinations, one token and runs longer than the window (the oldest slot is
overwritten within the call). The single-stream workload is compared on every head here; the
B=256 workloads the benchmark times are compared on every head in test_gpu_fullsize.py.
"""
import numpy as np
import pytest
import torch

import gated_deltanet_recurrent_02_amd as gdn
import oracle
from gated_deltanet_recurrent_02_amd import synth
from parity import (LOWRANK_STATE, check_lowrank, check_o, f64, gpu_lowrank, oracle_lowrank,
                    sample_heads, to_dev)

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
COMBOS = [("f32", "f32"), ("bf16", "f32"), ("bf16", "bf16"), ("f16", "f16"), ("f32", "bf16")]


def _announce(msg):
    print(f"[case] {msg}", flush=True)


@pytest.mark.parametrize("D", [16, 32, 64, 128])
@pytest.mark.parametrize("r", [8, 16, 32])
@pytest.mark.parametrize("act,sdt", COMBOS)
@pytest.mark.parametrize("B,H,T", [(3, 5, 1), (2, 3, 21)])
def test_small_shapes_full_compare(D, r, act, sdt, B, H, T):
    _announce(f"lowrank B={B} H={H} D={D} r={r} T={T} act={act} state={sdt}")
    x = synth.lowrank_inputs(B, H, D, T, r, act=act, state_dtype=sdt, seed=D + r + T)
    g, o = gpu_lowrank(x, scale=0.75)
    check_lowrank(g, o, oracle_lowrank(x, scale=0.75), DT[act], DT[sdt])


@pytest.mark.parametrize("r", [8, 16, 32])
def test_runs_longer_than_the_window_wrap_several_times(r):
    _announce(f"lowrank wrap B=2 H=3 D=32 r={r} T={3 * r + 5}")
    x = synth.lowrank_inputs(2, 3, 32, 3 * r + 5, r, act="bf16", alpha_shift=-2.0, seed=r)
    g, o = gpu_lowrank(x)
    check_lowrank(g, o, oracle_lowrank(x), torch.bfloat16, torch.float32)


@pytest.mark.parametrize("D", [16, 32, 64, 128])
@pytest.mark.parametrize("r", [8, 16, 32])
def test_empty_window_is_the_full_recurrence_until_it_fills(D, r):
    # From an empty window, as long as no write has left it, the low-rank state is the full
    # recurrence: o must match oracle_gdn_decode from S0 = 0 on the same tokens.
    _announce(f"lowrank empty window D={D} r={r} T={r}")
    x = synth.lowrank_inputs(2, 3, D, r, r, act="f32", window="empty", alpha_shift=-2.0, seed=3)
    g, o = gpu_lowrank(x)
    S0 = np.zeros((2, 3, D, D))
    _, o_full = oracle.gdn_decode(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["alpha"]),
                                  f64(x["beta"]), S0)
    check_o(f64(o), o_full, torch.float32)
    assert torch.equal(g["pos"].cpu(), torch.zeros(2, 3, dtype=torch.int32))


@pytest.mark.parametrize("sdt", ["f32", "bf16"])
def test_single_stream_workload_all_heads(sdt):
    # The B=1 workload on every head; the B=256 workloads are compared on every head in
    # test_gpu_fullsize.py.
    name = "lowrank_b1_h48_d128_r16_t1"
    _announce(f"{name} state={sdt}")
    x = synth.workload_inputs(name, state_dtype=sdt)
    g, o = gpu_lowrank(x)
    check_lowrank(g, o, oracle_lowrank(x), torch.bfloat16, DT[sdt])


def test_split_calls_equal_one_call_bitwise():
    # fp32 state: a call boundary stores and reloads exact values, so T tokens in one call and
    # the same tokens over two calls of 4 and 5 tokens agree bit for bit (each token's
    # arithmetic does not depend on how the call groups the tokens into rounds). Calls of fewer
    # than 4 tokens on an fp32 window take the vector kernel, whose key sums round
    # differently: see the next test.
    _announce("lowrank split calls B=2 H=5 D=128 r=16 T=9")
    x = synth.lowrank_inputs(2, 5, 128, 9, 16, act="bf16", seed=11)
    g1, o1 = gpu_lowrank(x)
    g2 = to_dev(x)
    outs = []
    for a, z in ((0, 4), (4, 9)):
        sl = slice(a, z)
        outs.append(gdn.lowrank_decode_step(*(g2[n][:, sl].contiguous()
                                              for n in ("q", "k", "v", "alpha", "beta")),
                                            g2["U"], g2["K"], g2["c"], g2["pos"]))
    torch.cuda.synchronize()
    assert torch.equal(o1, torch.cat(outs, dim=1))
    for n in LOWRANK_STATE:
        assert torch.equal(g1[n], g2[n]), n


@pytest.mark.parametrize("sdt", ["f32", "bf16"])
def test_split_calls_with_single_tokens_match_the_oracle(sdt):
    # Calls of 4, 1 and 4 tokens (the single-token call on the vector kernel, the others on the
    # matrix-core key products), each against the oracle run from the window the previous call
    # stored.
    _announce(f"lowrank split calls with a single token state={sdt}")
    x = synth.lowrank_inputs(2, 5, 128, 9, 16, act="bf16", state_dtype=sdt, seed=12)
    g = to_dev(x)
    win = {n: x[n] for n in LOWRANK_STATE}
    for a, z in ((0, 4), (4, 5), (5, 9)):
        part = {n: x[n][:, a:z].contiguous() for n in ("q", "k", "v", "alpha", "beta")}
        o = gdn.lowrank_decode_step(*(g[n][:, a:z].contiguous()
                                      for n in ("q", "k", "v", "alpha", "beta")),
                                    g["U"], g["K"], g["c"], g["pos"])
        torch.cuda.synchronize()
        ref = oracle_lowrank(dict(part, **win))
        check_lowrank({n: g[n] for n in LOWRANK_STATE}, o, ref, torch.bfloat16, DT[sdt])
        win = {n: g[n].cpu() for n in LOWRANK_STATE}


def test_pos_is_read_modulo_r():
    _announce("lowrank pos out of range")
    x = synth.lowrank_inputs(1, 4, 64, 3, 16, act="bf16", seed=5)
    x["pos"] = torch.tensor([[16 + 3, -1, 2 ** 31 - 1, 35]], dtype=torch.int32)
    g, o = gpu_lowrank(x)
    ref = oracle_lowrank(x)
    assert ref[3].tolist() == [[(3 + 3) % 16, (15 + 3) % 16, (15 + 3) % 16, (3 + 3) % 16]]
    check_lowrank(g, o, ref, torch.bfloat16, torch.float32)


def test_nan_stays_in_its_head():
    _announce("lowrank NaN isolation")
    x = synth.lowrank_inputs(2, 4, 128, 2, 16, act="f32", seed=6)
    x["v"][1, 0, 2, 5] = float("nan")
    g, o = gpu_lowrank(x)
    bad = torch.zeros(2, 4, dtype=torch.bool)
    bad[1, 2] = True
    for b in range(2):
        for h in range(4):
            finite = bool(torch.isfinite(o[b, :, h]).all()) and bool(torch.isfinite(g["U"][b, h]).all())
            assert finite != bool(bad[b, h]), (b, h)
    ref = oracle_lowrank(x, heads=[(0, 0), (1, 3)])
    got = {n: g[n].cpu()[[0, 1], [0, 3]] for n in LOWRANK_STATE}
    check_lowrank(got, o.cpu()[[0, 1], :, [0, 3]], ref, torch.float32, torch.float32)


def test_bitwise_deterministic():
    x = synth.lowrank_inputs(4, 6, 128, 3, 32, act="bf16", state_dtype="bf16", seed=8)
    g1, o1 = gpu_lowrank(x)
    g2, o2 = gpu_lowrank(x)
    assert torch.equal(o1, o2)
    for n in LOWRANK_STATE:
        assert torch.equal(g1[n], g2[n]), n


def test_graph_replays_match_eager():
    # Five rounds captured in one HIP graph, replayed three times with eager work between the
    # replays; every replay must equal the eager rounds on a copy of the same state.
    _announce("lowrank graph replay")
    x = synth.lowrank_inputs(8, 48, 128, 1, 16, act="bf16", seed=9)
    g = to_dev(x)
    e = to_dev(x)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        o = torch.empty_like(g["v"])
        gdn.lowrank_decode_step(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["U"], g["K"],
                                g["c"], g["pos"], o=o)  # warm-up round, mirrored below
    stream.synchronize()
    gdn.lowrank_decode_step(e["q"], e["k"], e["v"], e["alpha"], e["beta"], e["U"], e["K"],
                            e["c"], e["pos"])
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for _ in range(5):
            gdn.lowrank_decode_step(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["U"], g["K"],
                                    g["c"], g["pos"], o=o)
    for rep in range(3):
        graph.replay()
        torch.cuda.synchronize()
        for _ in range(5):
            oe = gdn.lowrank_decode_step(e["q"], e["k"], e["v"], e["alpha"], e["beta"], e["U"],
                                         e["K"], e["c"], e["pos"])
        torch.cuda.synchronize()
        assert torch.equal(o, oe), rep
        for n in LOWRANK_STATE:
            assert torch.equal(g[n], e[n]), (rep, n)


def test_empty_calls_change_nothing():
    x = synth.lowrank_inputs(2, 3, 64, 1, 8, act="bf16", seed=10)
    g = to_dev(x)
    before = {n: g[n].clone() for n in LOWRANK_STATE}
    e = lambda t: t[:, :0].contiguous()
    o = gdn.lowrank_decode_step(e(g["q"]), e(g["k"]), e(g["v"]), e(g["alpha"]), e(g["beta"]),
                                g["U"], g["K"], g["c"], g["pos"])
    torch.cuda.synchronize()
    assert o.shape == (2, 0, 3, 64)
    for n in LOWRANK_STATE:
        assert torch.equal(g[n], before[n]), n


def test_window_beyond_4_GiB_offsets():
    # B=6144 x H=48 heads of a 32-slot fp32 window: U and K hold 4.8 GB each, so byte offsets
    # pass 2^32. The window is drawn on the device from a seeded generator; sampled heads
    # (including the last) are read back before the call and compared with the oracle.
    _announce("lowrank B=6144 H=48 D=128 r=32 (2 x 4.8 GB window)")
    B, H, D, r = 6144, 48, 128, 32
    gen = torch.Generator(device="cuda").manual_seed(13)
    U = torch.randn(B, H, r, D, device="cuda", generator=gen).mul_(0.5)
    K = torch.randn(B, H, r, D, device="cuda", generator=gen)
    K /= K.norm(dim=-1, keepdim=True)
    c = torch.rand(B, H, r, device="cuda", generator=gen)
    pos = torch.randint(0, r, (B, H), device="cuda", generator=gen, dtype=torch.int32)
    x = synth.lowrank_inputs(B, H, D, 1, r, act="bf16", window="empty", seed=13)
    heads = sample_heads(B, H, 24, seed=13) + [(B - 1, 0), (B // 2, H - 1)]
    bt, ht = (torch.as_tensor(a) for a in np.asarray(heads).T)
    btd, htd = bt.cuda(), ht.cuda()
    before = {n: t[btd, htd].cpu() for n, t in (("U", U), ("K", K), ("c", c), ("pos", pos))}
    g = to_dev({n: x[n] for n in ("q", "k", "v", "alpha", "beta")})
    o = gdn.lowrank_decode_step(g["q"], g["k"], g["v"], g["alpha"], g["beta"], U, K, c, pos)
    torch.cuda.synchronize()
    got = {n: t[btd, htd].cpu() for n, t in (("U", U), ("K", K), ("c", c), ("pos", pos))}
    del U, K
    sel = lambda t: f64(t[bt, :, ht])[:, :, None]
    ref = oracle.gdn_lowrank_decode(sel(x["q"]), sel(x["k"]), sel(x["v"]), sel(x["alpha"]),
                                    sel(x["beta"]), f64(before["U"])[:, None],
                                    f64(before["K"])[:, None], f64(before["c"])[:, None],
                                    before["pos"].numpy()[:, None])
    ref = tuple(a[:, 0] for a in ref[:4]) + (ref[4][:, :, 0],)
    check_lowrank(got, o.cpu()[bt, :, ht], ref, torch.bfloat16, torch.float32)


@pytest.mark.parametrize("sdt", ["f32", "bf16"])
def test_identity_gate_replaces_only_the_oldest_slot(sdt):
    # alpha = 1, beta = 0: the write is exactly zero and no weight changes, so the call only
    # moves the oldest slot to (0, k, 1); every other slot, weight and key is untouched, bit
    # for bit.
    _announce(f"lowrank identity gate state={sdt}")
    x = synth.lowrank_inputs(3, 5, 128, 1, 16, act="bf16", state_dtype=sdt, seed=14)
    x["alpha"][:] = 1.0
    x["beta"][:] = 0.0
    g, o = gpu_lowrank(x)
    p = (x["pos"].long() & 15)
    B, H = p.shape
    for b in range(B):
        for h in range(H):
            pi = int(p[b, h])
            keep = [i for i in range(16) if i != pi]
            assert torch.equal(g["U"][b, h, keep].cpu(), x["U"][b, h, keep]), (b, h)
            assert torch.equal(g["K"][b, h, keep].cpu(), x["K"][b, h, keep]), (b, h)
            assert torch.equal(g["c"][b, h, keep].cpu(), x["c"][b, h, keep]), (b, h)
            assert bool((g["U"][b, h, pi] == 0).all()) and float(g["c"][b, h, pi]) == 1.0
            assert torch.equal(g["K"][b, h, pi].cpu(), x["k"][b, 0, h].to(DT[sdt]))
    assert torch.equal(g["pos"].cpu(), ((p + 1) % 16).int())
    check_lowrank(g, o, oracle_lowrank(x), torch.bfloat16, DT[sdt])


def test_zero_decay_keeps_only_the_new_write():
    # alpha = 0: every earlier write's weight becomes exactly 0, the new slot's 1, and the
    # write is beta v (S k is multiplied by 0), so o = scale beta (k . q) v.
    _announce("lowrank zero decay")
    x = synth.lowrank_inputs(2, 4, 64, 1, 8, act="f32", seed=15)
    x["alpha"][:] = 0.0
    g, o = gpu_lowrank(x, scale=0.5)
    p = (x["pos"].long() & 7)
    for b in range(2):
        for h in range(4):
            c = g["c"][b, h].cpu()
            expect = torch.zeros(8)
            expect[int(p[b, h])] = 1.0
            assert torch.equal(c, expect), (b, h)
    check_lowrank(g, o, oracle_lowrank(x, scale=0.5), torch.float32, torch.float32)


# Multi-token calls on a bf16 window with bf16 activations at D = 128 take each round of up to
# 8 tokens in matrix form (the round's writes through a triangular solve) when every round is
# full or nearly so (T >= 8 with T % 8 in {0, 6, 7}), else the per-token form; the cases below
# reach both forms, partial rounds, several rounds, wraps of the window within and across
# rounds, and the gate extremes.

@pytest.mark.parametrize("r", [16, 32])
@pytest.mark.parametrize("T", [2, 3, 4, 6, 7, 8, 9, 13, 14, 15, 16, 22, 53])
def test_rounds_on_bf16_windows(r, T):
    _announce(f"lowrank rounds B=2 H=3 D=128 r={r} T={T} act=bf16 state=bf16")
    x = synth.lowrank_inputs(2, 3, 128, T, r, act="bf16", state_dtype="bf16", alpha_shift=-1.0,
                             seed=100 + T + r)
    g, o = gpu_lowrank(x, scale=0.6)
    check_lowrank(g, o, oracle_lowrank(x, scale=0.6), torch.bfloat16, torch.bfloat16)


@pytest.mark.parametrize("T", [11, 14])
@pytest.mark.parametrize("window", ["filled", "empty"])
def test_rounds_gate_extremes(window, T):
    # Per head: alpha = 1 with beta = 0 (writes exactly zero, weights kept), alpha = 0 (earlier
    # writes drop out), alpha = 0 on every third token only, beta = 1, and negative alpha.
    _announce(f"lowrank rounds gate extremes window={window} T={T}")
    x = synth.lowrank_inputs(2, 5, 128, T, 16, act="bf16", state_dtype="bf16", window=window,
                             seed=31)
    x["alpha"][:, :, 0] = 1.0
    x["beta"][:, :, 0] = 0.0
    x["alpha"][:, :, 1] = 0.0
    x["alpha"][:, ::3, 2] = 0.0
    x["beta"][:, :, 3] = 1.0
    x["alpha"][:, :, 4] = -0.8
    g, o = gpu_lowrank(x)
    check_lowrank(g, o, oracle_lowrank(x), torch.bfloat16, torch.bfloat16)
    # alpha = 1, beta = 0: every write is zero and the untouched slots keep their weights.
    for b in range(2):
        p = int(x["pos"][b, 0]) & 15
        written = [(p + t) % 16 for t in range(T)]
        assert bool((g["U"][b, 0, written] == 0).all())
        kept = [i for i in range(16) if i not in written]
        assert torch.equal(g["c"][b, 0, kept].cpu(), x["c"][b, 0, kept])
        assert bool((g["c"][b, 0, written] == 1.0).all())


@pytest.mark.parametrize("T", [12, 14])
def test_rounds_nan_stays_in_its_head(T):
    # A NaN in one head's v at token 9 (the second round) poisons only that head, and there
    # only from its own round on: the products of the round form multiply it by the structural
    # zeros of T and M (0 * NaN = NaN), so the earlier tokens of its round are not asserted,
    # while the first round's outputs stay finite.
    _announce(f"lowrank rounds NaN isolation T={T}")
    x = synth.lowrank_inputs(2, 4, 128, T, 16, act="bf16", state_dtype="bf16", seed=32)
    x["v"][1, 9, 3, 7] = float("nan")
    g, o = gpu_lowrank(x)
    for b in range(2):
        for h in range(4):
            finite = bool(torch.isfinite(o[b, :, h]).all()) and bool(torch.isfinite(g["U"][b, h]).all())
            assert finite != (b == 1 and h == 3), (b, h)
    assert bool(torch.isfinite(o[1, :8, 3]).all())
    assert bool(torch.isnan(o[1, 9:, 3]).any(dim=-1).all())
    ref = oracle_lowrank(x, heads=[(0, 0), (1, 2)])
    got = {n: g[n].cpu()[[0, 1], [0, 2]] for n in LOWRANK_STATE}
    check_lowrank(got, o.cpu()[[0, 1], :, [0, 2]], ref, torch.bfloat16, torch.bfloat16)


def test_rounds_split_calls_continue_the_window():
    # 22 tokens as calls of 5, 1 and 16 tokens (round boundaries differ from one call's). The
    # window is stored in bf16 between calls, so the oracle runs call by call from the window
    # the previous call stored (U rounded to bf16; K is a copy of bf16 keys; c and pos exact).
    _announce("lowrank rounds split calls")
    x = synth.lowrank_inputs(2, 5, 128, 22, 16, act="bf16", state_dtype="bf16", seed=33)
    g = to_dev(x)
    win = {n: x[n] for n in LOWRANK_STATE}
    for a, z in ((0, 5), (5, 6), (6, 22)):
        part = {n: x[n][:, a:z].contiguous() for n in ("q", "k", "v", "alpha", "beta")}
        o = gdn.lowrank_decode_step(*(g[n][:, a:z].contiguous()
                                      for n in ("q", "k", "v", "alpha", "beta")),
                                    g["U"], g["K"], g["c"], g["pos"])
        torch.cuda.synchronize()
        ref = oracle_lowrank(dict(part, **win))
        check_lowrank({n: g[n] for n in LOWRANK_STATE}, o, ref, torch.bfloat16, torch.bfloat16)
        win = {n: g[n].cpu() for n in LOWRANK_STATE}


def test_rounds_graph_replays_match_eager():
    # Three 16-token calls captured in one HIP graph, replayed three times with eager work
    # between the replays; every replay must equal the eager calls on a copy of the state.
    _announce("lowrank rounds graph replay")
    x = synth.lowrank_inputs(4, 48, 128, 16, 16, act="bf16", state_dtype="bf16", seed=34)
    g = to_dev(x)
    e = to_dev(x)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        o = torch.empty_like(g["v"])
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for _ in range(3):
            gdn.lowrank_decode_step(g["q"], g["k"], g["v"], g["alpha"], g["beta"], g["U"], g["K"],
                                    g["c"], g["pos"], o=o)
    for rep in range(3):
        graph.replay()
        torch.cuda.synchronize()
        for _ in range(3):
            oe = gdn.lowrank_decode_step(e["q"], e["k"], e["v"], e["alpha"], e["beta"], e["U"],
                                         e["K"], e["c"], e["pos"])
        torch.cuda.synchronize()
        assert torch.equal(o, oe), rep
        for n in LOWRANK_STATE:
            assert torch.equal(g[n], e[n]), (rep, n)
