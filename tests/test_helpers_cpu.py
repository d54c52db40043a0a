"""CPU checks of the test helpers the full-size GPU parity tests rely on:
the threaded whole-batch oracle equals one oracle call, and the distance in
representable values counts neighbours as 1."""
import numpy as np
import torch

from speculative_decode_amd import workloads
from _helpers import bitwise_equal, format_steps, orc_spec, oracle_spec_parts


def test_oracle_spec_parts_equals_one_call():
    b = workloads.spec_batch(B=7, T=4, HK=1, HV=2, act="bf16", state="bf16",
                             q_lens=[4, 0, 2, 4, 1, 3, 4], acc_lo=0, acc_hi=4,
                             num_slots=30, seed=3)
    perm = np.random.default_rng(0).permutation(b.n_tok).astype(np.int32)
    b.spec_token_indx = torch.from_numpy(perm)
    pool, out = orc_spec(b)
    written, states, rows, outs = oracle_spec_parts(
        b.q, b.k, b.v, b.z, b.a, b.b, b.A_log, b.dt_bias, b.norm_weight, b.pool,
        b.cu_seqlens, b.spec_state_indices, b.num_accepted_tokens,
        token_indx=b.spec_token_indx, out_dtype=b.out_dtype, scale=b.scale,
        norm_eps=b.norm_eps, threads=3)
    lens = (b.cu_seqlens[1:] - b.cu_seqlens[:-1]).tolist()
    assert sorted(written) == sorted(s for i, L in enumerate(lens)
                                     for s in b.spec_state_indices[i, :L].tolist())
    assert bitwise_equal(states, pool[written])
    assert sorted(rows) == list(range(b.n_tok))
    assert bitwise_equal(outs, out[rows])


def test_format_steps_counts_neighbours():
    """Against numpy's nextafter for float16, and bit increments for bf16 and
    FP8: a neighbour is one step, the sign of zero none, and the two
    smallest subnormals of opposite sign two (zero lies between)."""
    x = np.random.default_rng(1).standard_normal(4096).astype(np.float16)
    up = np.nextafter(x, np.float16(np.inf))
    down = np.nextafter(x, np.float16(-np.inf))
    t = torch.from_numpy(x)
    assert (format_steps(t, torch.from_numpy(up)) == 1).all()
    assert (format_steps(t, torch.from_numpy(down)) == 1).all()
    assert (format_steps(torch.from_numpy(up), torch.from_numpy(down)) == 2).all()
    for dt, iv in ((torch.bfloat16, torch.int16), (torch.float8_e4m3fn, torch.int8)):
        y = torch.tensor([0.5, -3.0, 1e-2], dtype=torch.float32).to(dt)
        nxt = (y.view(iv).to(torch.int32) + 1).to(iv).view(dt)    # one magnitude step
        assert (format_steps(y, nxt) == 1).all()
        z = torch.zeros(2, dtype=dt)
        z[1] = -0.0
        assert (format_steps(z[:1], z[1:]) == 0).all()
        mpos = torch.tensor([1], dtype=iv).view(dt)
        mneg = (-mpos.float()).to(dt)
        assert (format_steps(mpos, mneg) == 2).all()
