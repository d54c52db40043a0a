"""Seeded synthetic inputs for the GDN speculative-decode update.

This module holds no arithmetic of the method: it only draws random numbers
and lays out metadata.  Tests, the benchmark and the smoke check all take
their inputs from here, so the GPU path and the CPU oracle always see the
same bytes.

Recipe (one ``numpy.random.Generator(PCG64(seed))`` per batch, drawn in this
order): q, k, v, z, a, b (standard normal, fp32), A_log ~ U(-1, 1),
dt_bias ~ U(-0.5, 0.5), norm_weight ~ U(0.5, 1.5), the state pool (normal
with the stated deviation, drawn slot by slot), the slot permutation,
num_accepted_tokens, and for mixed batches the order of the units.  Every
value is drawn in fp32 and rounded to nearest-even into its stated dtype.

The shapes follow the decode workloads on the vLLM PR reports: K = V = 128,
grouped heads HV = G * HK, at most 8 draft tokens per sequence, a state pool
of ``[num_slots, HV, V, K]`` with one slot per (sequence, draft token).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
       "f8": torch.float8_e4m3fn}


@dataclass
class GDNBatch:
    """One layer's worth of decode inputs (CPU tensors)."""
    name: str
    HK: int
    HV: int
    K: int
    V: int
    q: torch.Tensor            # [n_tok, HK, K]
    k: torch.Tensor            # [n_tok, HK, K]
    v: torch.Tensor            # [n_tok, HV, V]
    z: torch.Tensor            # [n_tok, HV, V]  output gate
    a: torch.Tensor            # [n_tok, HV]
    b: torch.Tensor            # [n_tok, HV]
    A_log: torch.Tensor        # [HV] fp32
    dt_bias: torch.Tensor      # [HV] fp32
    norm_weight: torch.Tensor  # [V] fp32
    pool: torch.Tensor         # [num_slots, HV, V, K]
    out_dtype: torch.dtype
    # speculative part (B sequences, row space of the spec call)
    cu_seqlens: torch.Tensor            # int32 [B+1]
    spec_state_indices: torch.Tensor    # int32 [B, T]
    num_accepted_tokens: torch.Tensor   # int32 [B]
    spec_token_indx: Optional[torch.Tensor] = None   # int32 [cu[B]] or None
    # non-speculative part (single-token, in-place)
    state_indices: Optional[torch.Tensor] = None     # int32 [N_ns]
    non_spec_token_indx: Optional[torch.Tensor] = None
    T: int = 0
    scale: float = field(default=0.0)
    norm_eps: float = 1e-5

    @property
    def n_tok(self) -> int:
        return self.q.shape[0]

    @property
    def num_seqs(self) -> int:
        return self.cu_seqlens.shape[0] - 1

    @property
    def num_non_spec(self) -> int:
        return 0 if self.state_indices is None else self.state_indices.shape[0]

    def spec_rows(self) -> int:
        return int(self.cu_seqlens[-1])

    def draft_tokens(self) -> int:
        """Rows processed by one step: spec rows plus non-spec entries."""
        ns = 0 if self.state_indices is None else int((self.state_indices >= 0).sum())
        return self.spec_rows() + ns

    def algorithmic_bytes(self) -> int:
        """Bytes one step must move: each active sequence reads its state once
        and writes one tile per token; each non-spec entry reads and writes one
        tile; every processed row moves q, k (per key head), v, z, out (per
        value head) and the two gate scalars; plus metadata and parameters."""
        s_state = self.pool.element_size()
        s_act = self.q.element_size()
        s_out = torch.empty((), dtype=self.out_dtype).element_size()
        tile = self.HV * self.K * self.V * s_state
        lens = (self.cu_seqlens[1:] - self.cu_seqlens[:-1]).clamp(min=0)
        active = lens > 0
        state = int(((1 + lens) * active).sum()) * tile
        ns = 0 if self.state_indices is None else int((self.state_indices >= 0).sum())
        state += 2 * ns * tile
        rows = self.draft_tokens()
        per_row = (2 * self.HK * self.K * s_act
                   + self.HV * self.V * (2 * s_act + s_out)
                   + 2 * self.HV * s_act)
        meta = 4 * (self.cu_seqlens.numel() + self.num_accepted_tokens.numel()
                    + int(active.sum()) * (self.T + 1))
        if self.spec_token_indx is not None:
            meta += 4 * self.spec_token_indx.numel()
        if self.state_indices is not None:
            meta += 4 * 2 * self.state_indices.numel()
        params = 4 * (2 * self.HV + self.V)
        return state + rows * per_row + meta + params


def _draw_act(rng, shape, dtype):
    x = rng.standard_normal(shape, dtype=np.float32)
    return torch.from_numpy(x).to(dtype)


def _draw_pool(rng, num_slots, HV, V, K, std, dtype):
    pool = torch.empty((num_slots, HV, V, K), dtype=dtype)
    for s in range(num_slots):
        x = rng.standard_normal((HV, V, K), dtype=np.float32) * np.float32(std)
        pool[s] = torch.from_numpy(x).to(dtype)
    return pool


def _common(rng, n_tok, HK, HV, K, V, act, num_slots, pool_std, state):
    q = _draw_act(rng, (n_tok, HK, K), act)
    k = _draw_act(rng, (n_tok, HK, K), act)
    v = _draw_act(rng, (n_tok, HV, V), act)
    z = _draw_act(rng, (n_tok, HV, V), act)
    a = _draw_act(rng, (n_tok, HV), act)
    b = _draw_act(rng, (n_tok, HV), act)
    A_log = torch.from_numpy(rng.uniform(-1.0, 1.0, HV).astype(np.float32))
    dt_bias = torch.from_numpy(rng.uniform(-0.5, 0.5, HV).astype(np.float32))
    norm_weight = torch.from_numpy(rng.uniform(0.5, 1.5, V).astype(np.float32))
    pool = _draw_pool(rng, num_slots, HV, V, K, pool_std, state)
    return q, k, v, z, a, b, A_log, dt_bias, norm_weight, pool


def spec_batch(*, B, T, HK, HV, K=128, V=128, act="bf16", state="bf16",
               out=None, num_slots=None, pool_std=0.05, acc_lo=0, acc_hi=None,
               q_lens=None, seed=0, name="spec") -> GDNBatch:
    """A pure speculative batch: B sequences of up to T draft tokens each.

    ``q_lens`` (default: all T) gives each sequence's row count; rows are laid
    out contiguously in sequence order.  ``spec_state_indices`` is a random
    permutation of the pool's slots reshaped to ``[B, T]`` (the first B*T
    entries when the pool is larger); num_accepted ~ U{acc_lo..acc_hi}.
    """
    acc_hi = T if acc_hi is None else acc_hi
    num_slots = B * T if num_slots is None else num_slots
    assert num_slots >= B * T
    lens = np.full(B, T, dtype=np.int64) if q_lens is None else np.asarray(q_lens, np.int64)
    assert lens.shape == (B,) and (lens <= T).all()
    cu = np.zeros(B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.maximum(lens, 0))
    n_tok = int(cu[-1])
    rng = np.random.Generator(np.random.PCG64(seed))
    act_t, state_t = _DT[act], _DT[state]
    q, k, v, z, a, b, A_log, dt_bias, w, pool = _common(
        rng, n_tok, HK, HV, K, V, act_t, num_slots, pool_std, state_t)
    perm = rng.permutation(num_slots).astype(np.int32)
    acc = rng.integers(acc_lo, acc_hi + 1, size=B).astype(np.int32)
    return GDNBatch(
        name=name, HK=HK, HV=HV, K=K, V=V, q=q, k=k, v=v, z=z, a=a, b=b,
        A_log=A_log, dt_bias=dt_bias, norm_weight=w, pool=pool,
        out_dtype=_DT[out or act], cu_seqlens=torch.from_numpy(cu),
        spec_state_indices=torch.from_numpy(perm[: B * T].reshape(B, T).copy()),
        num_accepted_tokens=torch.from_numpy(acc), T=T, scale=K ** -0.5)


def mixed_batch(*, n_non_spec, n_spec, T, HK, HV, K=128, V=128, act="bf16",
                state="bf16", out=None, pool_std=0.05, acc_lo=0, acc_hi=None,
                seed=0, name="mixed") -> GDNBatch:
    """Non-spec single tokens and spec sequences of T rows, in random order.

    The 'units' (singles and T-row blocks) are shuffled; rows are numbered in
    unit order.  Spec sequences are numbered in the order they appear, so
    ``spec_token_indx`` (their rows) is a non-identity gather index and
    ``non_spec_token_indx`` holds the remaining rows.  The pool has one slot
    per spec (sequence, token) plus one per non-spec entry, permuted.
    """
    acc_hi = T if acc_hi is None else acc_hi
    n_tok = n_non_spec + n_spec * T
    num_slots = n_tok
    rng = np.random.Generator(np.random.PCG64(seed))
    act_t, state_t = _DT[act], _DT[state]
    q, k, v, z, a, b, A_log, dt_bias, w, pool = _common(
        rng, n_tok, HK, HV, K, V, act_t, num_slots, pool_std, state_t)
    perm = rng.permutation(num_slots).astype(np.int32)
    acc = rng.integers(acc_lo, acc_hi + 1, size=n_spec).astype(np.int32)
    order = rng.permutation(n_non_spec + n_spec)
    spec_rows, ns_rows, row = [], [], 0
    for u in order:
        if u < n_non_spec:
            ns_rows.append(row)
            row += 1
        else:
            spec_rows.extend(range(row, row + T))
            row += T
    cu = np.arange(0, (n_spec + 1) * T, T, dtype=np.int32)
    return GDNBatch(
        name=name, HK=HK, HV=HV, K=K, V=V, q=q, k=k, v=v, z=z, a=a, b=b,
        A_log=A_log, dt_bias=dt_bias, norm_weight=w, pool=pool,
        out_dtype=_DT[out or act], cu_seqlens=torch.from_numpy(cu),
        spec_state_indices=torch.from_numpy(perm[: n_spec * T].reshape(n_spec, T).copy()),
        num_accepted_tokens=torch.from_numpy(acc),
        spec_token_indx=torch.tensor(spec_rows, dtype=torch.int32),
        state_indices=torch.from_numpy(perm[n_spec * T:].copy()),
        non_spec_token_indx=torch.tensor(ns_rows, dtype=torch.int32),
        T=T, scale=K ** -0.5)


# The decode workloads, named by shape.  "tiny" is small enough for the
# oracle to check whole in well under a second; "mtp_b128_bf16" (B=128, T=8,
# BF16 state) is the headline measurement.
CONFIGS = {
    "tiny": dict(kind="spec", B=2, T=3, HK=1, HV=8, act="f32", state="f32",
                 num_slots=8, pool_std=0.1, acc_lo=0, acc_hi=3, seed=0),
    "mtp_b32": dict(kind="spec", B=32, T=4, HK=4, HV=32, act="bf16", state="bf16",
                    acc_lo=1, acc_hi=4, seed=2),
    "mtp_b128_f32": dict(kind="spec", B=128, T=8, HK=4, HV=32, act="bf16", state="f32",
                         acc_lo=0, acc_hi=8, seed=3),
    "mtp_b128_bf16": dict(kind="spec", B=128, T=8, HK=4, HV=32, act="bf16", state="bf16",
                          acc_lo=0, acc_hi=8, seed=3),
    "mixed_b128": dict(kind="mixed", n_non_spec=64, n_spec=64, T=4, HK=4, HV=32,
                       act="bf16", state="bf16", acc_lo=0, acc_hi=4, seed=4),
    "large_b512_f16": dict(kind="spec", B=512, T=8, HK=16, HV=32, act="bf16", state="f16",
                           acc_lo=1, acc_hi=8, seed=5),
    "mtp_b128_f8": dict(kind="spec", B=128, T=8, HK=4, HV=32, act="bf16", state="f8",
                        acc_lo=0, acc_hi=8, seed=3),
    "decode_b128": dict(kind="mixed", n_non_spec=128, n_spec=0, T=1, HK=4, HV=32,
                        act="bf16", state="bf16", seed=6),
}

DESCRIPTIONS = {
    "tiny": "spec step B=2 T=3 HK=1 HV=8 K=V=128, fp32 activations, FP32 pool of 8 slots",
    "mtp_b32": "MTP decode B=32 T=4 HK=4 HV=32 K=V=128, bf16 activations, BF16 pool",
    "mtp_b128_f32": "MTP decode B=128 T=8 HK=4 HV=32 K=V=128, bf16 activations, FP32 pool, "
                    "acc 0..8",
    "mtp_b128_bf16": "MTP decode B=128 T=8 HK=4 HV=32 K=V=128, bf16 activations, BF16 pool, "
                     "acc 0..8",
    "mixed_b128": "mixed batch: 64 non-spec T=1 + 64 spec T=4, HK=4 HV=32 K=V=128, bf16, "
                  "BF16 pool",
    "large_b512_f16": "decode B=512 T=8 HK=16 HV=32 K=V=128, bf16 activations, FP16 pool",
    "mtp_b128_f8": "MTP decode B=128 T=8 HK=4 HV=32 K=V=128, bf16 activations, FP8 E4M3 pool, "
                   "acc 0..8",
    "decode_b128": "non-spec decode B=128 (one token each, slots updated in place) HK=4 HV=32 "
                   "K=V=128, bf16 activations, BF16 pool",
}


@dataclass
class PrefillBatch:
    """Chunked-prefill inputs (CPU tensors): B sequences of any length, rows
    contiguous in sequence order, one state slot per sequence."""
    name: str
    HK: int
    HV: int
    K: int
    V: int
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    z: torch.Tensor
    a: torch.Tensor
    b: torch.Tensor
    A_log: torch.Tensor
    dt_bias: torch.Tensor
    norm_weight: torch.Tensor
    pool: torch.Tensor
    out_dtype: torch.dtype
    cu_seqlens: torch.Tensor              # int32 [B+1]
    state_indices: torch.Tensor           # int32 [B]
    has_initial_state: Optional[torch.Tensor] = None   # int32 [B] or None (all)
    token_indx: Optional[torch.Tensor] = None
    chunk_size: int = 64
    scale: float = 0.0
    norm_eps: float = 1e-5

    @property
    def n_tok(self) -> int:
        return self.q.shape[0]

    @property
    def num_seqs(self) -> int:
        return self.cu_seqlens.shape[0] - 1

    def tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    def head_tokens(self) -> int:
        return self.tokens() * self.HV

    def algorithmic_bytes(self) -> int:
        """Per sequence and v-head with a slot: the state read once (when it
        has an initial state) and written once; per processed row: q, k per
        key head, v, z, out per value head and the two gates; plus metadata
        and parameters."""
        s_state = self.pool.element_size()
        s_act = self.q.element_size()
        s_out = torch.empty((), dtype=self.out_dtype).element_size()
        tile = self.HV * self.K * self.V * s_state
        lens = (self.cu_seqlens[1:] - self.cu_seqlens[:-1]).clamp(min=0)
        live = (lens > 0) & (self.state_indices >= 0)
        init = live.clone()
        if self.has_initial_state is not None:
            init &= self.has_initial_state != 0
        state = (int(live.sum()) + int(init.sum())) * tile
        rows = int((lens * live).sum())
        per_row = (2 * self.HK * self.K * s_act + self.HV * self.V * (2 * s_act + s_out)
                   + 2 * self.HV * s_act)
        meta = 4 * (self.cu_seqlens.numel() + self.state_indices.numel())
        if self.has_initial_state is not None:
            meta += 4 * self.has_initial_state.numel()
        return state + rows * per_row + meta + 4 * (2 * self.HV + self.V)

    def flops(self) -> int:
        """Arithmetic of the recurrence: per processed (row, v-head), the
        decay (K*V multiplies), S.k^ and S.q^ (2*K*V multiply-adds) and the
        rank-1 update (K*V multiply-adds): 7*K*V flop."""
        lens = (self.cu_seqlens[1:] - self.cu_seqlens[:-1]).clamp(min=0)
        live = (lens > 0) & (self.state_indices >= 0)
        return int((lens * live).sum()) * self.HV * 7 * self.K * self.V


def prefill_batch(*, lens, HK, HV, K=128, V=128, act="bf16", state="bf16", out=None,
                  num_slots=None, pool_std=0.05, chunk_size=64, init_frac=1.0, seed=0,
                  name="prefill") -> PrefillBatch:
    """Sequences of the given lengths, rows contiguous in order; slot of
    sequence b from a permutation of the pool; has_initial_state ~
    Bernoulli(init_frac) (None when init_frac is 1).  Draw order as for the
    decode batches (q, k, v, z, a, b, A_log, dt_bias, norm_weight, the pool
    slot by slot, the slot permutation), then has_initial_state."""
    lens = np.asarray(lens, dtype=np.int64)
    B = lens.shape[0]
    num_slots = B if num_slots is None else num_slots
    assert num_slots >= B
    cu = np.zeros(B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.maximum(lens, 0))
    rng = np.random.Generator(np.random.PCG64(seed))
    act_t, state_t = _DT[act], _DT[state]
    q, k, v, z, a, b, A_log, dt_bias, w, pool = _common(
        rng, int(cu[-1]), HK, HV, K, V, act_t, num_slots, pool_std, state_t)
    perm = rng.permutation(num_slots).astype(np.int32)
    hi = None
    if init_frac < 1.0:
        hi = torch.from_numpy((rng.random(B) < init_frac).astype(np.int32))
    return PrefillBatch(name=name, HK=HK, HV=HV, K=K, V=V, q=q, k=k, v=v, z=z, a=a, b=b,
                        A_log=A_log, dt_bias=dt_bias, norm_weight=w, pool=pool,
                        out_dtype=_DT[out or act], cu_seqlens=torch.from_numpy(cu),
                        state_indices=torch.from_numpy(perm[:B].copy()),
                        has_initial_state=hi, chunk_size=chunk_size, scale=K ** -0.5)


# Prefill workloads.  "prefill_b16_l2048": 16 sequences of 2048 tokens on the
# layer shape of the decode workloads, BF16 state rounded every 64 tokens.
PREFILL_CONFIGS = {
    "prefill_small": dict(lens=[200, 77, 0, 131], HK=2, HV=8, act="bf16", state="bf16",
                          chunk_size=32, init_frac=0.6, num_slots=6, seed=30),
    "prefill_b16_l2048": dict(lens=[2048] * 16, HK=4, HV=32, act="bf16", state="bf16",
                              chunk_size=64, seed=31),
    "prefill_ragged_b32": dict(lens=[64 * (1 + (7 * i) % 24) for i in range(32)], HK=4, HV=32,
                               act="bf16", state="bf16", chunk_size=64, init_frac=0.5, seed=32),
    "prefill_b8_l2048": dict(lens=[2048] * 8, HK=4, HV=32, act="bf16", state="bf16",
                             chunk_size=64, seed=33),
}

PREFILL_DESCRIPTIONS = {
    "prefill_small": "prefill B=4 (200, 77, 0, 131 tokens) HK=2 HV=8 K=V=128, bf16, BF16 "
                     "state, chunk 32",
    "prefill_b16_l2048": "prefill B=16 x 2048 tokens HK=4 HV=32 K=V=128, bf16 activations, "
                         "BF16 state rounded every 64 tokens",
    "prefill_ragged_b32": "prefill B=32, 64..1536 tokens, HK=4 HV=32 K=V=128, bf16, BF16 "
                          "state, chunk 64, half with an initial state",
    "prefill_b8_l2048": "prefill B=8 x 2048 tokens HK=4 HV=32 K=V=128, bf16 activations, "
                        "BF16 state rounded every 64 tokens (one unit per CU)",
}


def make_prefill(name: str, **overrides) -> PrefillBatch:
    cfg = dict(PREFILL_CONFIGS[name])
    cfg.update(overrides)
    return prefill_batch(name=name, **cfg)


@dataclass
class ConvBatch:
    """Inputs of the conv update that precedes the recurrent update (CPU
    tensors).  ``x`` holds the conv inputs (the packed q/k/v projection before
    the conv) of every row; ``cache`` is the wide rolling conv buffer,
    ``[num_lines, state_len, C]``; sequence b owns line ``conv_indices[b]``."""
    name: str
    x: torch.Tensor                     # [n_tok, C]
    weight: torch.Tensor                # [C, width] fp32
    bias: Optional[torch.Tensor]        # [C] fp32 or None
    cache: torch.Tensor                 # [num_lines, state_len, C]
    out_dtype: torch.dtype
    cu_seqlens: torch.Tensor            # int32 [B+1]
    conv_indices: torch.Tensor          # int32 [B]
    num_accepted_tokens: torch.Tensor   # int32 [B]
    token_indx: Optional[torch.Tensor] = None
    activation: str = "silu"
    T: int = 0

    @property
    def n_tok(self) -> int:
        return self.x.shape[0]

    @property
    def channels(self) -> int:
        return self.x.shape[1]

    @property
    def width(self) -> int:
        return self.weight.shape[1]

    @property
    def state_len(self) -> int:
        return self.cache.shape[1]

    @property
    def num_seqs(self) -> int:
        return self.cu_seqlens.shape[0] - 1

    def draft_tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    def algorithmic_bytes(self) -> int:
        """Per active sequence: read width-1 history positions and L inputs,
        write L outputs and width-2+L buffer positions; plus the weight and
        bias once and the metadata."""
        C, W = self.channels, self.width
        s_c, s_x = self.cache.element_size(), self.x.element_size()
        s_o = torch.empty((), dtype=self.out_dtype).element_size()
        lens = (self.cu_seqlens[1:] - self.cu_seqlens[:-1]).clamp(min=0)
        active = lens > 0
        n_act, rows = int(active.sum()), int(lens.sum())
        data = (n_act * (W - 1) * C * s_c + rows * C * s_x + rows * C * s_o
                + int(((W - 2 + lens) * active).sum()) * C * s_c)
        params = C * W * 4 + (0 if self.bias is None else C * 4)
        meta = 4 * (self.cu_seqlens.numel() + 2 * self.num_seqs)
        if self.token_indx is not None:
            meta += 4 * self.token_indx.numel()
        return data + params + meta


def conv_batch(*, B, T, C, width=4, state_len=None, dtype="bf16", out=None, num_lines=None,
               acc_lo=0, acc_hi=None, q_lens=None, bias=True, activation="silu", gather=False,
               seed=0, name="conv") -> ConvBatch:
    """B sequences of up to T draft rows over C channels.

    Draw order: x ~ N(0, 1), weight ~ U(-0.5, 0.5) ([C, width]), bias ~
    U(-0.5, 0.5), the buffer ~ N(0, 1) line by line, the line permutation,
    num_accepted ~ U{acc_lo..acc_hi}, and (gather=True) a row permutation used
    as token_indx.  state_len defaults to width - 2 + T, the least that holds
    a rewound history plus T new inputs.
    """
    acc_hi = T if acc_hi is None else acc_hi
    state_len = width - 2 + T if state_len is None else state_len
    num_lines = B if num_lines is None else num_lines
    assert num_lines >= B
    lens = np.full(B, T, dtype=np.int64) if q_lens is None else np.asarray(q_lens, np.int64)
    assert lens.shape == (B,) and (lens <= T).all()
    cu = np.zeros(B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.maximum(lens, 0))
    n_tok = int(cu[-1])
    rng = np.random.Generator(np.random.PCG64(seed))
    dt = _DT[dtype]
    x = _draw_act(rng, (n_tok, C), dt)
    weight = torch.from_numpy(rng.uniform(-0.5, 0.5, (C, width)).astype(np.float32))
    b = torch.from_numpy(rng.uniform(-0.5, 0.5, C).astype(np.float32)) if bias else None
    cache = torch.empty((num_lines, state_len, C), dtype=dt)
    for ln in range(num_lines):
        cache[ln] = _draw_act(rng, (state_len, C), dt)
    perm = rng.permutation(num_lines).astype(np.int32)
    acc = rng.integers(acc_lo, acc_hi + 1, size=B).astype(np.int32)
    tix = None
    if gather:
        tix = torch.from_numpy(rng.permutation(n_tok).astype(np.int32))
    return ConvBatch(name=name, x=x, weight=weight, bias=b, cache=cache,
                     out_dtype=_DT[out or dtype], cu_seqlens=torch.from_numpy(cu),
                     conv_indices=torch.from_numpy(perm[:B].copy()),
                     num_accepted_tokens=torch.from_numpy(acc), token_indx=tix,
                     activation=activation, T=T)


# Conv workloads.  C = 2*HK*K + HV*V channels (q, k and v of the GDN layer
# whose update follows), width 4, a buffer of width - 2 + T positions.
CONV_CONFIGS = {
    "conv_tiny": dict(B=3, T=3, C=40, width=4, dtype="f32", num_lines=6, acc_lo=0, acc_hi=3,
                      seed=10),
    "conv_mtp_b128": dict(B=128, T=8, C=2 * 4 * 128 + 32 * 128, width=4, dtype="bf16",
                          num_lines=256, acc_lo=0, acc_hi=8, seed=11),
}

CONV_DESCRIPTIONS = {
    "conv_tiny": "conv update B=3 T=3 C=40 width 4, fp32, 6 buffer lines",
    "conv_mtp_b128": "conv update B=128 T=8 C=5120 (HK=4 HV=32 K=V=128) width 4, bf16 "
                     "inputs/buffer/outputs, SiLU, acc 0..8",
}


def make_conv(name: str, **overrides) -> ConvBatch:
    cfg = dict(CONV_CONFIGS[name])
    cfg.update(overrides)
    return conv_batch(name=name, **cfg)


def make(name: str, **overrides) -> GDNBatch:
    cfg = dict(CONFIGS[name])
    cfg.update(overrides)
    kind = cfg.pop("kind")
    if kind == "mixed":
        return mixed_batch(name=name, **cfg)
    return spec_batch(name=name, **cfg)


@dataclass
class PostConvBatch:
    """One decode step from the packed projections through the conv update
    with rewind and the recurrent update (CPU tensors).

    ``x`` [n_tok, C] is the packed q/k/v projection before the conv, C =
    2 HK K + HV V in the order q, k, v; the conv writes its output into one
    buffer of the same shape, which the recurrent update reads as three
    strided views.  ``zba`` [n_tok, HV V + 2 HV] packs the output gate z and
    the gate inputs b, a, read as views too (never split into copies).
    Spec sequence b owns conv line ``conv_lines[b]``; single-token entry i
    owns ``ns_conv_lines[i]``; both take their rows through the gather
    indices when those are given."""
    name: str
    HK: int
    HV: int
    K: int
    V: int
    x: torch.Tensor                     # [n_tok, C]
    zba: torch.Tensor                   # [n_tok, HV V + 2 HV]
    conv_weight: torch.Tensor           # [C, width] fp32
    conv_bias: torch.Tensor             # [C] fp32
    conv_cache: torch.Tensor            # [num_lines, state_len, C]
    A_log: torch.Tensor
    dt_bias: torch.Tensor
    norm_weight: torch.Tensor
    pool: torch.Tensor                  # [num_slots, HV, V, K]
    cu_seqlens: torch.Tensor            # int32 [B+1]
    spec_state_indices: torch.Tensor    # int32 [B, T]
    num_accepted_tokens: torch.Tensor   # int32 [B]
    conv_lines: torch.Tensor            # int32 [B]
    spec_token_indx: Optional[torch.Tensor] = None
    state_indices: Optional[torch.Tensor] = None
    ns_conv_lines: Optional[torch.Tensor] = None
    non_spec_token_indx: Optional[torch.Tensor] = None
    T: int = 0
    scale: float = 0.0
    norm_eps: float = 1e-5

    @property
    def n_tok(self) -> int:
        return self.x.shape[0]

    @property
    def num_seqs(self) -> int:
        return self.cu_seqlens.shape[0] - 1


def postconv_batch(*, n_spec, T, n_non_spec=0, HK, HV, K=128, V=128, act="bf16",
                   state="bf16", width=4, acc_lo=0, acc_hi=None, gather=None, pool_std=0.05,
                   seed=0, name="postconv") -> PostConvBatch:
    """A decode step of n_spec sequences of T draft rows and n_non_spec
    single tokens.  With gather (default: when there are single tokens) the
    units are laid out in random order and both parts reach their rows
    through gather indices, as in a mixed batch.

    Draw order: x, zba ~ N(0, 1); conv weight, bias ~ U(-0.5, 0.5); A_log ~
    U(-1, 1), dt_bias ~ U(-0.5, 0.5), norm_weight ~ U(0.5, 1.5); the conv
    buffer ~ N(0, 1) line by line; the pool ~ N(0, pool_std) slot by slot;
    the line permutation, the slot permutation, num_accepted ~
    U{acc_lo..acc_hi}; the unit order."""
    acc_hi = T if acc_hi is None else acc_hi
    gather = n_non_spec > 0 if gather is None else gather
    C = 2 * HK * K + HV * V
    n_tok = n_spec * T + n_non_spec
    num_lines = n_spec + n_non_spec
    num_slots = n_spec * T + n_non_spec
    state_len = width - 2 + T
    rng = np.random.Generator(np.random.PCG64(seed))
    act_t = _DT[act]
    x = _draw_act(rng, (n_tok, C), act_t)
    zba = _draw_act(rng, (n_tok, HV * V + 2 * HV), act_t)
    cw = torch.from_numpy(rng.uniform(-0.5, 0.5, (C, width)).astype(np.float32))
    cb = torch.from_numpy(rng.uniform(-0.5, 0.5, C).astype(np.float32))
    A_log = torch.from_numpy(rng.uniform(-1.0, 1.0, HV).astype(np.float32))
    dt_bias = torch.from_numpy(rng.uniform(-0.5, 0.5, HV).astype(np.float32))
    w = torch.from_numpy(rng.uniform(0.5, 1.5, V).astype(np.float32))
    cache = torch.empty((num_lines, state_len, C), dtype=act_t)
    for ln in range(num_lines):
        cache[ln] = _draw_act(rng, (state_len, C), act_t)
    pool = _draw_pool(rng, num_slots, HV, V, K, pool_std, _DT[state])
    lines = rng.permutation(num_lines).astype(np.int32)
    slots = rng.permutation(num_slots).astype(np.int32)
    acc = rng.integers(acc_lo, acc_hi + 1, size=n_spec).astype(np.int32)
    spec_rows, ns_rows = list(range(n_spec * T)), list(range(n_spec * T, n_tok))
    if gather:
        spec_rows, ns_rows, row = [], [], 0
        for u in rng.permutation(n_spec + n_non_spec):
            if u < n_non_spec:
                ns_rows.append(row)
                row += 1
            else:
                spec_rows.extend(range(row, row + T))
                row += T
    cu = np.arange(0, (n_spec + 1) * T, T, dtype=np.int32)
    ns = n_non_spec > 0
    return PostConvBatch(
        name=name, HK=HK, HV=HV, K=K, V=V, x=x, zba=zba, conv_weight=cw, conv_bias=cb,
        conv_cache=cache, A_log=A_log, dt_bias=dt_bias, norm_weight=w, pool=pool,
        cu_seqlens=torch.from_numpy(cu),
        spec_state_indices=torch.from_numpy(slots[:n_spec * T].reshape(n_spec, T).copy()),
        num_accepted_tokens=torch.from_numpy(acc),
        conv_lines=torch.from_numpy(lines[:n_spec].copy()),
        spec_token_indx=torch.tensor(spec_rows, dtype=torch.int32) if gather else None,
        state_indices=torch.from_numpy(slots[n_spec * T:].copy()) if ns else None,
        ns_conv_lines=torch.from_numpy(lines[n_spec:].copy()) if ns else None,
        non_spec_token_indx=torch.tensor(ns_rows, dtype=torch.int32) if ns else None,
        T=T, scale=K ** -0.5)
