"""gdn_prefill_noalloc (the chunked prefill with the library's fixed device scratch instead of a
caller's workspace) against gdn_prefill on the same inputs, through the C ABI.

Both run the same kernels on the same data, so o and the state must agree bit for bit. Two
calls in a row: the first fills nearly the whole 64 MiB scratch (one 48-head sequence of
10,000 tokens, 30,000 records of 2176 bytes), the second is smaller and ragged, so stale
records of the first call lie beyond what the second writes. A call past the limit is refused
on the host with GDN_ERR_UNSUPPORTED and changes nothing.
"""
import pytest
import torch

import gated_deltanet_recurrent_02_amd as gdn
from gated_deltanet_recurrent_02_amd import synth
from parity import to_dev

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 64 << 20


def _announce(msg):
    print(f"[case] {msg}", flush=True)


def _both(x, scale=1.0):
    """(o, state) from gdn_prefill with its own workspace and from gdn_prefill_noalloc."""
    a, b = to_dev(x), to_dev(x)
    o_ws = gdn.prefill(a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["state"], scale=scale)
    o_na = torch.empty_like(b["v"])
    gdn.prefill_noalloc(b["q"], b["k"], b["v"], b["alpha"], b["beta"], b["state"], o_na,
                        scale=scale)
    torch.cuda.synchronize()
    return (o_ws, a["state"]), (o_na, b["state"])


def _bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


@pytest.mark.parametrize("sdt", ["f32", "bf16"])
def test_noalloc_equals_prefill_on_two_calls(sdt):
    cases = [(1, 48, 10000, 0.8), (2, 5, 37, 0.6)]
    for B, H, T, scale in cases:
        need = gdn.prefill_workspace_size(B, T, H, 128, 128)
        assert need <= SCRATCH_BYTES
        _announce(f"prefill_noalloc B={B} H={H} T={T} state={sdt} ({need} scratch bytes)")
        x = synth.decode_inputs(B, H, 128, T, act="bf16", state_dtype=sdt, alpha_shift=-2.0,
                                state_std=0.3, seed=T)
        (o_ws, S_ws), (o_na, S_na) = _both(x, scale)
        assert torch.equal(_bits(o_ws), _bits(o_na)), f"o differs at B={B} H={H} T={T}"
        assert torch.equal(_bits(S_ws), _bits(S_na)), f"state differs at B={B} H={H} T={T}"


def test_noalloc_refuses_more_than_its_scratch():
    B, H, T = 1, 48, 10400   # 48 * 650 records of 2176 bytes = 67,891,200 > 64 MiB
    assert gdn.prefill_workspace_size(B, T, H, 128, 128) > SCRATCH_BYTES
    _announce(f"prefill_noalloc over the limit B={B} H={H} T={T}")
    x = to_dev(synth.decode_inputs(B, H, 128, T, act="bf16", seed=3))
    S0 = x["state"].clone()
    o = torch.zeros_like(x["v"])
    with pytest.raises(gdn.GDNError) as e:
        gdn.prefill_noalloc(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["state"], o)
    assert e.value.status == 2 and "fixed scratch" in str(e.value)
    torch.cuda.synchronize()
    assert torch.equal(x["state"], S0) and not o.any()
