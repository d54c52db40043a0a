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
