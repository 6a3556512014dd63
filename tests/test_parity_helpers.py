"""CPU tests of the parity helpers' own arithmetic (no GPU): as_stored, the rounding of an fp64
state to its storage type, against torch's casts from fp32 (a single round to nearest even,
ties included) and against the formats' definitions at their edges."""
import numpy as np
import torch

from parity import as_stored, check_o


def _fp32_values(n=200_000, seed=0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(n) * np.exp2(rng.integers(-140, 20, n))
    # exact ties of bf16 (8 significant bits) and fp16 (11), and values on either side
    m = rng.integers(1 << 7, 1 << 8, 2000).astype(np.float64)
    ties = np.concatenate([(m + 0.5) * 2.0 ** -8, (m * 8 + 0.5) * 2.0 ** -11])
    ties = np.concatenate([ties, -ties, np.nextafter(ties, 0), np.nextafter(ties, 2)])
    return np.concatenate([x, ties, [0.0, -0.0, 1.0, 2.0 ** -130, 2.0 ** -20]]).astype(np.float32)


def test_as_stored_matches_torch_casts_of_fp32_values():
    x = _fp32_values()
    for dtype in (torch.bfloat16, torch.float16):
        want = torch.from_numpy(x).to(dtype).double().numpy()
        got = as_stored(x.astype(np.float64), dtype)
        fin = np.isfinite(want)  # fp16 overflows are outside the helper's range
        assert np.array_equal(got[fin], want[fin]), dtype
    assert np.array_equal(as_stored(x.astype(np.float64), torch.float32), x.astype(np.float64))


def test_as_stored_rounds_fp64_directly():
    # 1 + 2^-8 + 2^-30 lies just above a bf16 tie: direct rounding goes up, while rounding to
    # fp32 first would make it a tie and round to even (down).
    x = np.array([1.0 + 2.0 ** -8 + 2.0 ** -30, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8])
    assert np.array_equal(as_stored(x, torch.bfloat16),
                          [1.0 + 2.0 ** -7, 1.0, 1.0 + 2.0 ** -6])
    # fp16 subnormals are multiples of 2^-24
    y = np.array([2.0 ** -24 * 0.5, 2.0 ** -24 * 0.75, 2.0 ** -24 * 2.5, 2.0 ** -15])
    assert np.array_equal(as_stored(y, torch.float16), [0.0, 2.0 ** -24, 2.0 * 2.0 ** -24, 2.0 ** -15])


def test_check_o_accepts_every_correctly_rounded_output():
    # check_o must admit the exact value rounded once to the output type, subnormals included
    # (fp16 below 2^-14 rounds to multiples of 2^-24), and reject one unit more.
    rng = np.random.default_rng(3)
    # token vectors from 2^-22 (fp16 subnormals) to 2^1 in scale
    ref = rng.standard_normal((2, 5, 3, 64)) * np.exp2(rng.integers(-22, 2, (2, 5, 3, 1)))
    for dtype in (torch.bfloat16, torch.float16):
        check_o(as_stored(ref, dtype), ref, dtype)
    # 1.5 2^-25 rounds to 2^-24 (error 2^-25): admitted; a whole unit more is not
    tiny = np.full((1, 1, 1, 4), 1.5 * 2.0 ** -25)
    check_o(as_stored(tiny, torch.float16), tiny, torch.float16)
    off = as_stored(tiny, torch.float16) + 2.0 ** -24
    try:
        check_o(off, tiny, torch.float16)
    except AssertionError:
        pass
    else:
        raise AssertionError("one unit beyond the rounding passed")
