"""The library's state-store conversion (gdn_cast_to_state, the same code
every kernel uses at a state store) against the oracle's rounding, bit for
bit, in every state format: nearest-even, subnormals, exact ties, the FP8
saturation point, infinities and NaN."""
import numpy as np
import pytest
import torch

import oracle
from speculative_decode_amd import ops

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ops.load_library()
    return torch.device("cuda:0")


def sweep(dtype):
    rng = np.random.default_rng(7)
    fi = torch.finfo(dtype)
    lo = int(np.log2(fi.tiny)) - 12
    hi = int(np.log2(fi.max)) + 2
    x = rng.standard_normal(20000) * np.exp2(rng.integers(lo, hi, 20000).astype(np.float64))
    parts = [x]
    if dtype != torch.float32:
        # exact midpoints between neighbouring representable values: the
        # next value up is the bit pattern plus one
        g = torch.from_numpy(np.abs(x[:4000])).to(torch.float32).to(dtype)
        ib = torch.uint8 if g.element_size() == 1 else torch.int16
        nxt = (g.view(ib).to(torch.int32) + 1).to(ib).view(dtype)
        mid = (g.to(torch.float64) + nxt.to(torch.float64)).numpy() / 2
        mid = mid[np.isfinite(mid)]
        parts += [mid, -mid]
    parts.append([0.0, -0.0, np.inf, -np.inf, np.nan, 448.0, 463.99, 464.0, 464.01, -500.0,
                  2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -10, 65504.0, 65520.0, 1e38])
    with np.errstate(over="ignore"):        # beyond fp32: becomes inf, also a case
        return np.concatenate([np.asarray(p, dtype=np.float64) for p in parts]).astype(
            np.float32)


@pytest.mark.parametrize("dtype", [torch.float8_e4m3fn, torch.bfloat16, torch.float16,
                                   torch.float32])
def test_cast_matches_oracle(dev, dtype):
    x = sweep(dtype)
    got = ops.cast_to_state(torch.from_numpy(x).to(dev), dtype).cpu().to(torch.float64).numpy()
    ref = oracle.round_to(dtype, x.astype(np.float64))
    both_nan = np.isnan(got) & np.isnan(ref)
    bad = ~both_nan & (got != ref)
    assert not bad.any(), (x[bad][:8], got[bad][:8], ref[bad][:8])
    # signed zeros keep their sign
    z = np.signbit(got[x == 0]) == np.signbit(x[x == 0])
    assert z.all()
