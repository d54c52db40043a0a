"""Pins of the conv-update oracle against facts fixed by the PR reports and by
the mathematics, so that a wrong rewind offset, a reversed or shifted window,
a dropped bias, a misplaced activation or a wrong write-back fails one of them.

The decisive pin is streaming equivalence: a causal conv applied step by step
through the rolling buffer -- with drafts of any length and any acceptance --
must give, for every draft token, what a single depthwise conv1d (torch's
F.conv1d, the routine the #46090 CPU path calls) gives over the accepted input
stream followed by the current drafts.  Page references: #46090 (CPU DFlash
spec decode for GDN: implementation breakdown items 1-2, gdn_attention.py
excerpt), #51674 (fused post-conv MTP decode: implementation breakdown item 3).
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from speculative_decode_amd import workloads

F64 = torch.float64


def _conv_ref(stream, weight, bias, activation):
    """Depthwise causal conv1d over a [n, C] stream by torch, float64; returns
    the n - width + 1 outputs whose window lies inside the stream."""
    C, W = weight.shape
    inp = torch.as_tensor(stream, dtype=F64).T.unsqueeze(0)          # [1, C, n]
    y = F.conv1d(inp, torch.as_tensor(weight, dtype=F64).unsqueeze(1),
                 None if bias is None else torch.as_tensor(bias, dtype=F64), groups=C)
    y = y[0].T                                                        # [n - W + 1, C]
    if activation == "silu":
        y = F.silu(y)
    return y


def _spec(x, weight, bias, cache, lens, lines, acc, *, token_indx=None, out=None,
          activation="silu", out_dtype=F64):
    cu = torch.zeros(len(lens) + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(lens, dtype=torch.int32).clamp(min=0), 0)
    return oracle.conv_spec_update(x, weight, bias, cache, cu,
                                   torch.tensor(lines, dtype=torch.int32),
                                   torch.tensor(acc, dtype=torch.int32),
                                   token_indx=token_indx, out=out, out_dtype=out_dtype,
                                   activation=activation)


@pytest.mark.parametrize("width,T,activation,with_bias", [
    (4, 5, "silu", True), (4, 8, "none", False), (2, 3, "silu", False), (3, 6, "none", True)])
def test_stream_equivalence_under_rewind(width, T, activation, with_bias):
    """Step by step through one buffer line, with random draft lengths and
    acceptances (0 included, which keeps one draft like 1), every output
    equals the direct conv over accepted stream ++ drafts."""
    rng = np.random.default_rng(100 + width * 10 + T)
    C = 5
    S = width - 2 + T
    weight = rng.uniform(-1, 1, (C, width))
    bias = rng.uniform(-1, 1, C) if with_bias else None
    cache = torch.from_numpy(rng.standard_normal((2, S, C)))
    acc = int(rng.integers(1, S - width + 3))            # initial rewind offset acc - 1
    stream = cache[0, acc - 1: acc - 1 + width - 1].numpy().copy()
    for _ in range(8):
        L = int(rng.integers(1, T + 1))
        drafts = rng.standard_normal((L, C))
        before = cache.clone()
        cache, out = _spec(torch.from_numpy(drafts), torch.from_numpy(weight),
                           None if bias is None else torch.from_numpy(bias), cache,
                           [L], [0], [acc], activation=activation)
        ref = _conv_ref(np.vstack([stream[-(width - 1):], drafts]) if width > 1 else drafts,
                        weight, bias, activation)
        assert ref.shape == (L, C)
        np.testing.assert_allclose(out.numpy(), ref.numpy(), rtol=1e-12, atol=1e-12)
        assert torch.equal(cache[1], before[1])            # the other line is untouched
        acc = int(rng.integers(0, L + 1))
        stream = np.vstack([stream, drafts[: max(acc, 1)]])


def test_nonspec_decode_is_a_plain_causal_conv():
    """With a buffer of exactly width - 1 positions, successive single-token
    decode calls reproduce the direct conv of the whole token stream."""
    rng = np.random.default_rng(7)
    C, W, n = 4, 4, 12
    weight, bias = rng.uniform(-1, 1, (C, W)), rng.uniform(-1, 1, C)
    stream = rng.standard_normal((W - 1 + n, C))
    cache = torch.from_numpy(stream[: W - 1].copy()).unsqueeze(0)
    outs = []
    for i in range(n):
        x = torch.from_numpy(stream[W - 1 + i: W + i].copy())
        cache, out = oracle.conv_decode_update(x, torch.from_numpy(weight),
                                               torch.from_numpy(bias), cache,
                                               torch.tensor([0], dtype=torch.int32),
                                               out_dtype=F64)
        outs.append(out[0])
    ref = _conv_ref(stream, weight, bias, "silu")
    np.testing.assert_allclose(torch.stack(outs).numpy(), ref.numpy(), rtol=1e-12, atol=1e-12)
    assert torch.equal(cache[0], torch.from_numpy(stream[-(W - 1):]))


def test_decode_equals_spec_with_one_token_accepted_once():
    b = workloads.make_conv("conv_tiny")
    n = b.num_seqs
    x = b.x[:n]
    lines = b.conv_indices
    c1, o1 = oracle.conv_decode_update(x, b.weight, b.bias, b.cache, lines)
    c2, o2 = oracle.conv_spec_update(x, b.weight, b.bias, b.cache,
                                     torch.arange(n + 1, dtype=torch.int32), lines,
                                     torch.ones(n, dtype=torch.int32))
    assert torch.equal(c1, c2) and torch.equal(o1, o2)


def test_acc_zero_behaves_as_one():
    b = workloads.make_conv("conv_tiny")
    acc0 = torch.zeros_like(b.num_accepted_tokens)
    acc1 = torch.ones_like(b.num_accepted_tokens)
    r0 = oracle.conv_spec_update(b.x, b.weight, b.bias, b.cache, b.cu_seqlens, b.conv_indices, acc0)
    r1 = oracle.conv_spec_update(b.x, b.weight, b.bias, b.cache, b.cu_seqlens, b.conv_indices, acc1)
    assert torch.equal(r0[0], r1[0]) and torch.equal(r0[1], r1[1])


def test_touched_positions_lines_and_rows():
    """Only positions [0, width - 2 + L) of active lines change; skipped
    sequences (L = 0) and unused lines keep every byte; output rows of
    skipped sequences keep their contents."""
    lens = [3, 0, 2, 1]
    b = workloads.conv_batch(B=4, T=3, C=16, width=4, dtype="bf16", num_lines=7, q_lens=lens,
                             seed=3)
    sentinel = torch.full((b.n_tok + 2, b.channels), 7.0, dtype=b.out_dtype)
    cache, out = oracle.conv_spec_update(b.x, b.weight, b.bias, b.cache, b.cu_seqlens,
                                         b.conv_indices, b.num_accepted_tokens, out=sentinel)
    W = b.width
    active = {int(b.conv_indices[i]): L for i, L in enumerate(lens) if L > 0}
    for ln in range(b.cache.shape[0]):
        changed = (cache[ln] != b.cache[ln]).any(dim=1).nonzero().flatten().tolist()
        if ln in active:
            assert torch.equal(cache[ln, W - 2 + active[ln]:], b.cache[ln, W - 2 + active[ln]:])
            assert set(changed) <= set(range(W - 2 + active[ln]))
        else:
            assert changed == []
    assert torch.equal(out[b.n_tok:], sentinel[b.n_tok:])       # rows no sequence owns


def test_decode_negative_line_is_padding():
    b = workloads.make_conv("conv_tiny")
    n = b.num_seqs
    lines = b.conv_indices.clone()
    lines[1] = -1
    sentinel = torch.full((n, b.channels), -3.0, dtype=b.out_dtype)
    cache, out = oracle.conv_decode_update(b.x[:n], b.weight, b.bias, b.cache, lines,
                                           out=sentinel)
    assert torch.equal(out[1], sentinel[1])
    assert torch.equal(cache[int(b.conv_indices[1])], b.cache[int(b.conv_indices[1])])


def test_gather_alignment():
    """A non-identity token_indx equals running on pre-gathered rows and
    scattering the outputs back; ignoring the index gives something else."""
    b = workloads.conv_batch(B=3, T=4, C=8, dtype="f32", seed=5, gather=True)
    tix = b.token_indx.long()
    c1, o1 = oracle.conv_spec_update(b.x, b.weight, b.bias, b.cache, b.cu_seqlens,
                                     b.conv_indices, b.num_accepted_tokens, token_indx=b.token_indx)
    c2, o2g = oracle.conv_spec_update(b.x[tix], b.weight, b.bias, b.cache, b.cu_seqlens,
                                      b.conv_indices, b.num_accepted_tokens)
    o2 = torch.empty_like(o2g)
    o2[tix] = o2g
    assert torch.equal(c1, c2) and torch.equal(o1, o2)
    c3, o3 = oracle.conv_spec_update(b.x, b.weight, b.bias, b.cache, b.cu_seqlens,
                                     b.conv_indices, b.num_accepted_tokens)
    assert not torch.equal(o3, o1)


def test_linearity_without_bias_and_activation():
    b = workloads.conv_batch(B=3, T=4, C=8, dtype="f32", bias=False, activation="none", seed=6)
    x, cache = b.x.to(F64), b.cache.to(F64)
    c1, o1 = oracle.conv_spec_update(x, b.weight, None, cache, b.cu_seqlens, b.conv_indices,
                                     b.num_accepted_tokens, activation="none")
    c2, o2 = oracle.conv_spec_update(4 * x, b.weight, None, 4 * cache, b.cu_seqlens,
                                     b.conv_indices, b.num_accepted_tokens, activation="none")
    assert torch.equal(4 * o1, o2) and torch.equal(4 * c1, c2)


def test_identity_kernel_passes_inputs_through():
    """weight = e_{width-1}, no bias, no activation: each output is its own
    input, rounded once into the output format."""
    b = workloads.conv_batch(B=2, T=3, C=8, dtype="bf16", out="f16", seed=8)
    w = torch.zeros_like(b.weight)
    w[:, -1] = 1.0
    _, out = oracle.conv_spec_update(b.x, w, None, b.cache, b.cu_seqlens, b.conv_indices,
                                     b.num_accepted_tokens, activation="none")
    assert torch.equal(out, b.x.to(torch.float16))   # torch's one RNE step bf16 -> f16
