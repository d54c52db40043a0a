"""GPU parity of the post-conv decode step, the fused path of the vLLM PR
#51674 report (实现拆解 item 3): the causal conv1d update with rewind runs
first, keyed by num_accepted_tokens, and the recurrent update then reads the
packed projection without splitting it into q/k/v/z/b/a copies.

Here that chain is: gdn_conv_spec_update (and gdn_conv_decode_update for the
single tokens of a mixed batch) writes ONE conv output buffer [n_tok, C],
C = 2 HK K + HV V; q, k and v are strided views of it, z, b and a strided
views of one packed gate projection; gdn_spec_decode_update /
gdn_mixed_decode_update run on those views.  The oracle runs the same chain
(conv oracle, then the recurrent oracle on the q/k/v of ITS conv output), and
the results are compared at the bars of the two separate suites:
  * conv buffer: bit-exact;
  * conv output: relative L2 < 5e-4 over the processed rows;
  * state: element-wise atol = rtol = 3e-2 (the report's state bar, for an
    FP32 pool too: each side's recurrent update reads its own conv output,
    and an element the two convs round to neighbouring bf16 values moves the
    state far more than the 1e-5 FP32 bar of the separate suite allows),
    every written slot; every other slot byte-identical;
  * output: relative L2 < 5e-4 over the processed rows, the others zero.
"""
import pytest
import torch

import oracle
from speculative_decode_amd import ops, workloads
from _helpers import compare_states_on_device, oracle_spec_parts, rel_l2, slots_touched

OUT_REL_L2 = 5e-4
CHAIN_STATE_TOL = (3e-2, 3e-2)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    ops.load_library()
    return torch.device("cuda:0")


def qkv_views(y, pb):
    n, D = y.shape[0], pb.K
    q = y[:, :pb.HK * D].view(n, pb.HK, D)
    k = y[:, pb.HK * D:2 * pb.HK * D].view(n, pb.HK, D)
    v = y[:, 2 * pb.HK * D:].view(n, pb.HV, pb.V)
    return q, k, v


def zba_views(zba, pb):
    n, HV, V = zba.shape[0], pb.HV, pb.V
    return (zba[:, :HV * V].view(n, HV, V), zba[:, HV * V + HV:], zba[:, HV * V:HV * V + HV])


def spec_rows(pb):
    n = int(pb.cu_seqlens[-1])
    return pb.spec_token_indx.tolist() if pb.spec_token_indx is not None else list(range(n))


def processed(pb):
    rows = spec_rows(pb)
    if pb.non_spec_token_indx is not None:
        rows += pb.non_spec_token_indx.tolist()
    return sorted(rows)


def run_gpu(pb, dev):
    d = lambda t: None if t is None else t.to(dev)   # noqa: E731
    x, zba = d(pb.x), d(pb.zba)
    cache, pool = d(pb.conv_cache).clone(), d(pb.pool).clone()
    y = torch.zeros_like(x)
    ops.conv_spec_update(x, d(pb.conv_weight), d(pb.conv_bias), cache, d(pb.cu_seqlens),
                         d(pb.conv_lines), d(pb.num_accepted_tokens),
                         token_indx=d(pb.spec_token_indx), out=y, activation="silu",
                         max_q_len=pb.T)
    if pb.state_indices is not None:
        ops.conv_decode_update(x, d(pb.conv_weight), d(pb.conv_bias), cache,
                               d(pb.ns_conv_lines), token_indx=d(pb.non_spec_token_indx),
                               out=y, activation="silu")
    q, k, v = qkv_views(y, pb)
    z, a, b = zba_views(zba, pb)
    assert not q.is_contiguous() and not z.is_contiguous() and not a.is_contiguous()
    before = pool.clone()
    out = torch.zeros((pb.n_tok, pb.HV, pb.V), dtype=pb.x.dtype, device=dev)
    ops.forward_core(q, k, v, z, a, b, d(pb.A_log), d(pb.dt_bias), d(pb.norm_weight), pool,
                     spec_cu_seqlens=d(pb.cu_seqlens),
                     spec_state_indices=d(pb.spec_state_indices),
                     num_accepted_tokens=d(pb.num_accepted_tokens),
                     spec_token_indx=d(pb.spec_token_indx),
                     non_spec_state_indices=d(pb.state_indices),
                     non_spec_token_indx=d(pb.non_spec_token_indx), out=out,
                     scale=pb.scale, norm_eps=pb.norm_eps, max_q_len=pb.T)
    torch.cuda.synchronize()
    return cache.cpu(), y.cpu(), before, pool, out.cpu()


def oracle_conv(pb):
    c, y = oracle.conv_spec_update(pb.x, pb.conv_weight, pb.conv_bias, pb.conv_cache,
                                   pb.cu_seqlens, pb.conv_lines, pb.num_accepted_tokens,
                                   token_indx=pb.spec_token_indx, out_dtype=pb.x.dtype,
                                   activation="silu")
    if pb.state_indices is not None:
        c, y = oracle.conv_decode_update(pb.x, pb.conv_weight, pb.conv_bias, c,
                                         pb.ns_conv_lines, token_indx=pb.non_spec_token_indx,
                                         out=y, activation="silu")
    return c, y


def check_conv(pb, gc, gy, oc, oy):
    assert torch.equal(gc, oc), "conv buffer differs from the oracle"
    rows = processed(pb)
    err = rel_l2(gy[rows].double().numpy(), oy[rows].double().numpy())
    assert err < OUT_REL_L2, f"conv output rel L2 {err:.3e}"
    other = [r for r in range(pb.n_tok) if r not in set(rows)]
    assert (gy[other] == 0).all()
    return err


def test_postconv_chain_full_size(dev):
    """B = 128 sequences of 8 drafts, HK = 4, HV = 32 (C = 5,120 conv
    channels), bf16 activations and conv buffer, BF16 pool: the
    conv_mtp_b128 / mtp_b128_bf16 shapes, every sequence checked."""
    pb = workloads.postconv_batch(n_spec=128, T=8, HK=4, HV=32, act="bf16", state="bf16",
                                  acc_lo=0, acc_hi=8, seed=51, name="postconv_b128")
    print(f"[postconv_b128] n_tok={pb.n_tok} C={pb.x.shape[1]} pool={tuple(pb.pool.shape)}",
          flush=True)
    gc, gy, before, gpool, gout = run_gpu(pb, dev)
    oc, oy = oracle_conv(pb)
    cerr = check_conv(pb, gc, gy, oc, oy)
    q, k, v = (t.contiguous() for t in qkv_views(oy, pb))
    z, a, b = (t.contiguous() for t in zba_views(pb.zba, pb))
    written, states, rows, outs = oracle_spec_parts(
        q, k, v, z, a, b, pb.A_log, pb.dt_bias, pb.norm_weight, pb.pool, pb.cu_seqlens,
        pb.spec_state_indices, pb.num_accepted_tokens, out_dtype=pb.x.dtype, scale=pb.scale,
        norm_eps=pb.norm_eps)
    assert slots_touched(before, gpool) == sorted(written)
    compare_states_on_device(gpool, written, states, pb.pool.dtype, "postconv_b128",
                             step_rule=False, tol=CHAIN_STATE_TOL)
    err = rel_l2(gout[rows].double().numpy(), outs.double().numpy())
    assert err < OUT_REL_L2, f"output rel L2 {err:.3e}"
    print(f"[postconv_b128] conv out rel L2 {cerr:.2e}, out rel L2 {err:.2e}", flush=True)


@pytest.mark.parametrize("state", ["bf16", "f32"])
def test_postconv_chain_mixed_gathered(dev, state):
    """A mixed batch: 16 single tokens and 16 sequences of 4 drafts in random
    unit order, both parts gathered; the conv's spec and single-token entries
    write one buffer, and one launch runs the recurrent update on its views."""
    pb = workloads.postconv_batch(n_spec=16, T=4, n_non_spec=16, HK=4, HV=32, act="bf16",
                                  state=state, acc_lo=0, acc_hi=4, seed=52)
    pb.state_indices[3] = -1                 # a padded single token: nothing changes
    pb.ns_conv_lines[3] = -1
    gc, gy, before, gpool, gout = run_gpu(pb, dev)
    oc, oy = oracle_conv(pb)
    check_conv(pb, gc, gy, oc, oy)
    q, k, v = (t.contiguous() for t in qkv_views(oy, pb))
    z, a, b = (t.contiguous() for t in zba_views(pb.zba, pb))
    f = dict(out_dtype=pb.x.dtype, scale=pb.scale, norm_eps=pb.norm_eps)
    po, oo = oracle.spec_update(q, k, v, z, a, b, pb.A_log, pb.dt_bias, pb.norm_weight, pb.pool,
                                pb.cu_seqlens, pb.spec_state_indices, pb.num_accepted_tokens,
                                token_indx=pb.spec_token_indx, **f)
    po, oo = oracle.decode_update(q, k, v, z, a, b, pb.A_log, pb.dt_bias, pb.norm_weight, po,
                                  pb.state_indices, token_indx=pb.non_spec_token_indx, out=oo,
                                  **f)
    gp = gpool.cpu()
    want = sorted(set(pb.spec_state_indices.flatten().tolist())
                  | {s for s in pb.state_indices.tolist() if s >= 0})
    assert slots_touched(pb.pool, gp) == slots_touched(pb.pool, po) == want
    compare_states_on_device(gpool, want, po[want], pb.pool.dtype, f"postconv_mixed_{state}",
                             step_rule=False, tol=CHAIN_STATE_TOL)
    rows = [r for r in processed(pb) if r != int(pb.non_spec_token_indx[3])]
    err = rel_l2(gout[rows].double().numpy(), oo[rows].double().numpy())
    assert err < OUT_REL_L2, f"output rel L2 {err:.3e}"
    other = [r for r in range(pb.n_tok) if r not in set(rows)]
    assert (gout[other] == 0).all()
