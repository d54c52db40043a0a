"""Shared test helpers: running the oracle on a GDNBatch, recovering the raw
read-out o from a gated-RMSNorm output, and the parity metrics."""
from __future__ import annotations

import numpy as np
import torch

import oracle
from speculative_decode_amd import workloads


def tiny(*, K=4, V=4, HK=1, HV=2, B=2, T=3, state="f32", act="f32", seed=0,
         acc_lo=0, acc_hi=None, q_lens=None, num_slots=None, pool_std=0.3):
    return workloads.spec_batch(B=B, T=T, HK=HK, HV=HV, K=K, V=V, act=act,
                                state=state, out=act, seed=seed,
                                acc_lo=acc_lo, acc_hi=acc_hi, q_lens=q_lens,
                                num_slots=num_slots, pool_std=pool_std)


def with_pool_dtype(batch, dtype):
    batch.pool = batch.pool.to(dtype)
    return batch


def orc_spec(bt, *, pool=None, out=None, out_dtype=None, **over):
    f = dict(q=bt.q, k=bt.k, v=bt.v, z=bt.z, a=bt.a, b=bt.b, A_log=bt.A_log,
             dt_bias=bt.dt_bias, norm_weight=bt.norm_weight,
             cu_seqlens=bt.cu_seqlens, spec_state_indices=bt.spec_state_indices,
             num_accepted_tokens=bt.num_accepted_tokens,
             token_indx=bt.spec_token_indx, scale=bt.scale, norm_eps=bt.norm_eps)
    f.update(over)
    pool = bt.pool if pool is None else pool
    return oracle.spec_update(f.pop("q"), f.pop("k"), f.pop("v"), f.pop("z"),
                              f.pop("a"), f.pop("b"), f.pop("A_log"),
                              f.pop("dt_bias"), f.pop("norm_weight"), pool,
                              f.pop("cu_seqlens"), f.pop("spec_state_indices"),
                              f.pop("num_accepted_tokens"), out=out,
                              out_dtype=out_dtype or bt.out_dtype, **f)


def orc_decode(bt, state_indices, *, token_indx=None, pool=None, out=None,
               out_dtype=None, **over):
    f = dict(q=bt.q, k=bt.k, v=bt.v, z=bt.z, a=bt.a, b=bt.b, A_log=bt.A_log,
             dt_bias=bt.dt_bias, norm_weight=bt.norm_weight, scale=bt.scale,
             norm_eps=bt.norm_eps)
    f.update(over)
    pool = bt.pool if pool is None else pool
    return oracle.decode_update(f.pop("q"), f.pop("k"), f.pop("v"), f.pop("z"),
                                f.pop("a"), f.pop("b"), f.pop("A_log"),
                                f.pop("dt_bias"), f.pop("norm_weight"), pool,
                                state_indices, token_indx=token_indx, out=out,
                                out_dtype=out_dtype or bt.out_dtype, **f)


def silu(x):
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def recover_o(y, w, z, eps):
    """Invert y = o / sqrt(mean_V(o^2) + eps) * w * silu(z) for o.

    With u = y / (w silu z): mean(u^2) = ms / (ms + eps), so
    ms = eps * m / (1 - m) and o = u * sqrt(ms + eps)."""
    u = np.asarray(y, np.float64) / (np.asarray(w, np.float64) * silu(z))
    m = np.mean(u * u, axis=-1, keepdims=True)
    ms = eps * m / (1.0 - m)
    return u * np.sqrt(ms + eps)


def rel_l2(x, ref) -> float:
    x = np.asarray(x, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (den if den > 0 else 1.0))


def slots_touched(before: torch.Tensor, after: torch.Tensor):
    """(slot) indices whose bytes changed, as a sorted list."""
    nb = before.view(before.shape[0], -1)
    na = after.view(after.shape[0], -1)
    if before.dtype in (torch.bfloat16, torch.float16):
        nb, na = nb.view(torch.int16), na.view(torch.int16)
    elif before.dtype == torch.float32:
        nb, na = nb.view(torch.int32), na.view(torch.int32)
    else:
        nb, na = nb.view(torch.int64), na.view(torch.int64)
    return sorted(torch.nonzero((nb != na).any(dim=1)).flatten().tolist())


def bitwise_equal(x: torch.Tensor, y: torch.Tensor) -> bool:
    if x.shape != y.shape or x.dtype != y.dtype:
        return False
    xb = x.contiguous().view(torch.uint8)
    yb = y.contiguous().view(torch.uint8)
    return bool(torch.equal(xb, yb))


def oracle_spec_parts(q, k, v, z, a, b, A_log, dt_bias, norm_weight, pool, cu_seqlens,
                      spec_state_indices, num_accepted_tokens, *, token_indx=None,
                      out_dtype, scale, norm_eps, threads=16):
    """oracle.spec_update over EVERY sequence of a large batch.

    The sequences are split into ``threads`` contiguous parts, each run as
    its own oracle call on a host thread (ctypes releases the interpreter
    lock during the C call; the parts share nothing).  A part gets only its
    own rows and a pool of the slots its sequences read or write, so the
    float64 copies stay bounded.  Returns ``(written, states, rows, outs)``:
    the slots written (every spec_state_indices[b, t], t < L_b), the oracle's
    state at each ``[n, HV, V, K]`` in the pool dtype, the processed output
    rows and the oracle's output at each ``[m, HV, V]``."""
    from concurrent.futures import ThreadPoolExecutor

    cu = [int(x) for x in cu_seqlens.tolist()]
    si = spec_state_indices.tolist()
    B = len(cu) - 1
    n = max(1, min(threads, B))
    bounds = [B * i // n for i in range(n + 1)]
    oracle.round_to(torch.float32, [0.0])          # load the library before the threads

    def part(lo, hi):
        g = list(range(cu[lo], cu[hi]))
        rows = [int(token_indx[x]) for x in g] if token_indx is not None else g
        slots = sorted({s for r in si[lo:hi] for s in r})
        remap = {s: i for i, s in enumerate(slots)}
        si_c = torch.tensor([[remap[s] for s in r] for r in si[lo:hi]], dtype=torch.int32)
        ridx = torch.tensor(rows, dtype=torch.long)
        sub = [x[ridx] for x in (q, k, v, z, a, b)]
        cu_c = torch.tensor([c - cu[lo] for c in cu[lo:hi + 1]], dtype=torch.int32)
        p, o = oracle.spec_update(*sub, A_log, dt_bias, norm_weight, pool[slots], cu_c, si_c,
                                  num_accepted_tokens[lo:hi], out_dtype=out_dtype,
                                  scale=scale, norm_eps=norm_eps)
        wr = [si[bi][t] for bi in range(lo, hi) for t in range(max(cu[bi + 1] - cu[bi], 0))]
        widx = torch.tensor([remap[s] for s in wr], dtype=torch.long)
        return wr, p[widx], rows, o

    with ThreadPoolExecutor(n) as ex:
        res = list(ex.map(lambda i: part(bounds[i], bounds[i + 1]), range(n)))
    written = [s for r in res for s in r[0]]
    rows = [x for r in res for x in r[2]]
    return written, torch.cat([r[1] for r in res]), rows, torch.cat([r[3] for r in res])


def _ordered(bits: torch.Tensor, nbits: int) -> torch.Tensor:
    """Sign-magnitude float bit patterns as integers ordered like the values
    (+0 and -0 both map to 0), so that adjacent representable values differ
    by exactly 1."""
    x = bits.to(torch.int32) & ((1 << nbits) - 1)
    mag = x & ((1 << (nbits - 1)) - 1)
    return torch.where((x >> (nbits - 1)) != 0, -mag, mag)


def format_steps(x: torch.Tensor, y: torch.Tensor) -> torch.Tensor:
    """Distance in representable values between two tensors of one 8- or
    16-bit float format (elementwise, int32): 0 where the bits agree up to
    the sign of zero, 1 for neighbouring values."""
    assert x.dtype == y.dtype and x.element_size() in (1, 2)
    nbits = 8 * x.element_size()
    view = torch.int8 if nbits == 8 else torch.int16
    return (_ordered(x.view(view), nbits) - _ordered(y.view(view), nbits)).abs()


# Parity bars of the state (vLLM PR #51674 report, 实现拆解 item 5: state
# atol/rtol 3e-2), tightened for FP32 state; FP8 E4M3: one unit in the last
# place -- spacing 2^-9 below 2^-6, |x| 2^-3 above.
STATE_TOL = {torch.float32: 1e-5, torch.bfloat16: 3e-2, torch.float16: 3e-2}
F8_TOL = (2.0 ** -9, 2.0 ** -3)

# Stored tiles of a 8/16-bit pool against the oracle's rounding.  The kernel
# carries the state in FP32 and the oracle in double, so where the exact
# value lies within the FP32 error of a rounding boundary the two round to
# neighbouring values; elsewhere the bits agree.  Measured at full size
# (every stored element of mtp_b128_bf16, large_b512_f16, mtp_b128_f8): 6.8e-5
# of BF16, 3.4e-4 of FP16 and 8e-7 of FP8 elements differ, each by one step.
# The bounds below are about three times those shares.  Where a stored value
# is tiny next to the tile's other values, the FP32 error of the cancellation
# that produced it can span more than one step: the one-step rule applies
# above STEP_FLOOR, the element-wise bar below it.
STEP_FLOOR = {torch.bfloat16: 2.0 ** -12, torch.float16: 2.0 ** -10,
              torch.float8_e4m3fn: 2.0 ** -6}
STEP_SHARE_BOUND = {torch.bfloat16: 2e-4, torch.float16: 1e-3,
                    torch.float8_e4m3fn: 5e-6}


def compare_states_on_device(gpu_pool, written, states, dtype, what, *, chunk=64,
                             step_rule=True, tol=None):
    """Every written slot against the oracle, on the device in chunks:
    the element-wise bar, and for 8/16-bit pools the share of elements that
    differ from the oracle's rounding and by how many representable steps
    (asserted with step_rule; reported only when the two sides' inputs may
    themselves differ by a rounding, as after a conv computed on each).
    ``tol`` = (atol, rtol) replaces the bar of the pool dtype.""" 
    dev = gpu_pool.device
    atol, rtol = tol or (F8_TOL if dtype == torch.float8_e4m3fn else (STATE_TOL[dtype],) * 2)
    worst, differ, total, far = -np.inf, 0, 0, 0
    for i in range(0, len(written), chunk):
        idx = torch.tensor(written[i:i + chunk], dtype=torch.long, device=dev)
        g = gpu_pool[idx]
        o = states[i:i + chunk].to(dev)
        gd, od = g.double(), o.double()
        assert torch.isfinite(gd).all(), f"{what}: non-finite state"
        worst = max(worst, float(((gd - od).abs() - (atol + rtol * od.abs())).max()))
        if g.element_size() < 4:
            steps = format_steps(g, o)
            differ += int((steps > 0).sum())
            far += int(((steps > 1) & (od.abs() >= STEP_FLOOR[dtype])).sum())
        total += g.numel()
    assert worst <= 0, f"{what}: state mismatch, worst excess {worst:.3e}"
    if dtype in STEP_FLOOR and total:
        share = differ / total
        print(f"[{what}] stored elements differing from the oracle's rounding: {differ} of "
              f"{total} ({share:.2e}); more than one step above {STEP_FLOOR[dtype]:g}: {far}",
              flush=True)
        if step_rule:
            assert far == 0, f"{what}: {far} stored elements more than one step from the oracle"
            assert share <= STEP_SHARE_BOUND[dtype], \
                f"{what}: {share:.2e} of stored elements differ"


