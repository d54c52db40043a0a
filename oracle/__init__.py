"""CPU oracle of the GDN speculative-decode state update and of the conv
update that precedes it -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls anything here, and nothing
here imports the product package.

The arithmetic lives in ``gdn_oracle.c`` and ``conv_oracle.c`` (plain serial
C, every operation in double); this module only marshals torch/numpy arrays
into them:
inputs of any float dtype are upcast exactly to float64, the C code rounds to
the storage format at each slot/output write, and the results are cast back
to the caller's dtypes (exact, because the values are already representable).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRCS = [os.path.join(_HERE, "gdn_oracle.c"), os.path.join(_HERE, "conv_oracle.c")]
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

FMT_F32, FMT_F16, FMT_BF16, FMT_F64, FMT_F8E4M3 = 0, 1, 2, 3, 4
_FMT = {torch.float32: FMT_F32, torch.float16: FMT_F16,
        torch.bfloat16: FMT_BF16, torch.float64: FMT_F64,
        torch.float8_e4m3fn: FMT_F8E4M3}
_ERR = {1: "bad argument", 2: "index out of range", 3: "out of memory"}

_lib = None


def build() -> str:
    """Compile liboracle.so with gcc (no FMA contraction, no fast-math)."""
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-o", tmp] + _SRCS + ["-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    d, i32, i64, vp = ctypes.c_double, ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    lib.orc_round.restype = d
    lib.orc_round.argtypes = [ctypes.c_int, d]
    common_head = [vp] * 9 + [vp, ctypes.c_int, vp, ctypes.c_int, i64, i64]
    lib.orc_spec_update.restype = ctypes.c_int
    lib.orc_spec_update.argtypes = common_head + [vp, i32, vp, i64, vp, vp,
                                                  i32, i32, i32, i32, d, d]
    lib.orc_decode_update.restype = ctypes.c_int
    lib.orc_decode_update.argtypes = common_head + [vp, i32, vp,
                                                    i32, i32, i32, i32, d, d]
    lib.orc_prefill_update.restype = ctypes.c_int
    lib.orc_prefill_update.argtypes = common_head + [vp, i32, vp, vp, vp, i32,
                                                     i32, i32, i32, i32, d, d]
    lib.orc_conv_update.restype = ctypes.c_int
    lib.orc_conv_update.argtypes = [vp, vp, ctypes.c_int, vp, ctypes.c_int, i64, i32, i64,
                                    i32, i32, vp, vp, i32, vp, i32, vp, vp, vp]
    _lib = lib
    return lib


def round_to(dtype: torch.dtype, x) -> np.ndarray:
    """Element-wise orc_round (nearest, ties to even) into ``dtype``'s format."""
    lib = _load()
    fmt = _FMT[dtype]
    xs = np.asarray(x, dtype=np.float64).ravel()
    return np.array([lib.orc_round(fmt, float(e)) for e in xs]).reshape(np.shape(x))


def _f64(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        return np.ascontiguousarray(t.detach().cpu().to(torch.float64).numpy())
    return np.ascontiguousarray(np.asarray(t, dtype=np.float64))


def _i32(t):
    if t is None:
        return None
    if isinstance(t, torch.Tensor):
        t = t.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(t, dtype=np.int32))


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _prepare(q, k, v, z, a, b, A_log, dt_bias, norm_weight, pool, out, out_dtype):
    n_tok, HK, K = q.shape
    HV, V = v.shape[1], v.shape[2]
    assert k.shape == (n_tok, HK, K) and z.shape == (n_tok, HV, V)
    assert a.shape == (n_tok, HV) and b.shape == (n_tok, HV)
    assert pool.shape[1:] == (HV, V, K)
    if out is None:
        out = torch.zeros((n_tok, HV, V), dtype=out_dtype or z.dtype)
    arrs = [_f64(x) for x in (q, k, v, z, a, b, A_log, dt_bias, norm_weight)]
    # pool and out are written by the C code: always work on private copies
    return (arrs, _f64(out).copy(), out.dtype, _f64(pool).copy(),
            (n_tok, HK, HV, K, V))


class PreparedCall:
    """One oracle call with its arguments already marshalled: ``run()``
    executes only the C function (so that it can be timed alone) and
    ``result()`` converts the written pool and output back to tensors."""

    def __init__(self, fn_name, args, keep, what, finish):
        self._fn_name, self._args, self._what, self._finish = fn_name, args, what, finish
        self._keep = keep           # the arrays the marshalled pointers refer to

    def run(self):
        rc = getattr(_load(), self._fn_name)(*self._args)
        if rc:
            raise ValueError(f"oracle {self._what}: {_ERR.get(rc, rc)}")
        return self

    def result(self):
        return self._finish()


def _tensors_back(pool64, pool_dtype, out64, out_dtype):
    return lambda: (torch.from_numpy(pool64).to(pool_dtype), torch.from_numpy(out64).to(out_dtype))


def prepare_spec_update(q, k, v, z, a, b, A_log, dt_bias, norm_weight, pool,
                        cu_seqlens, spec_state_indices, num_accepted_tokens, *,
                        token_indx=None, out=None, out_dtype=None, scale=None,
                        norm_eps=1e-5) -> PreparedCall:
    """spec_update's arguments marshalled for the C call (see spec_update)."""
    arrs, out64, odt, pool64, (n_tok, HK, HV, K, V) = _prepare(
        q, k, v, z, a, b, A_log, dt_bias, norm_weight, pool, out, out_dtype)
    cu = _i32(cu_seqlens)
    si = _i32(spec_state_indices)
    na = _i32(num_accepted_tokens)
    ti = _i32(token_indx)
    B = cu.shape[0] - 1
    stride = si.shape[1] if si.ndim == 2 else max(1, si.shape[0] // max(B, 1))
    scale = K ** -0.5 if scale is None else scale
    args = (*[_p(x) for x in arrs], _p(out64), _FMT[odt], _p(pool64), _FMT[pool.dtype],
            pool.shape[0], n_tok, _p(cu), B, _p(si), stride, _p(na), _p(ti),
            HK, HV, K, V, float(scale), float(norm_eps))
    keep = (arrs, cu, si, na, ti, out64, pool64)
    return PreparedCall("orc_spec_update", args, keep,
                        "spec_update", _tensors_back(pool64, pool.dtype, out64, odt))


def spec_update(q, k, v, z, a, b, A_log, dt_bias, norm_weight, pool,
                cu_seqlens, spec_state_indices, num_accepted_tokens, *,
                token_indx=None, out=None, out_dtype=None, scale=None,
                norm_eps=1e-5):
    """Speculative update; returns ``(pool_after, out_after)`` as new tensors.

    ``pool`` is ``[num_slots, HV, V, K]``; ``spec_state_indices`` is
    ``[B, spec_stride]``; ``out`` (default zeros) supplies the rows that are
    not processed.  Inputs are not modified.
    """
    return prepare_spec_update(q, k, v, z, a, b, A_log, dt_bias, norm_weight, pool, cu_seqlens,
                               spec_state_indices, num_accepted_tokens, token_indx=token_indx,
                               out=out, out_dtype=out_dtype, scale=scale,
                               norm_eps=norm_eps).run().result()


def prepare_decode_update(q, k, v, z, a, b, A_log, dt_bias, norm_weight, pool,
                          state_indices, *, token_indx=None, out=None, out_dtype=None,
                          scale=None, norm_eps=1e-5) -> PreparedCall:
    """decode_update's arguments marshalled for the C call (see decode_update)."""
    arrs, out64, odt, pool64, (n_tok, HK, HV, K, V) = _prepare(
        q, k, v, z, a, b, A_log, dt_bias, norm_weight, pool, out, out_dtype)
    si = _i32(state_indices)
    ti = _i32(token_indx)
    scale = K ** -0.5 if scale is None else scale
    args = (*[_p(x) for x in arrs], _p(out64), _FMT[odt], _p(pool64), _FMT[pool.dtype],
            pool.shape[0], n_tok, _p(si), si.shape[0], _p(ti),
            HK, HV, K, V, float(scale), float(norm_eps))
    keep = (arrs, si, ti, out64, pool64)
    return PreparedCall("orc_decode_update", args, keep,
                        "decode_update", _tensors_back(pool64, pool.dtype, out64, odt))


def decode_update(q, k, v, z, a, b, A_log, dt_bias, norm_weight, pool,
                  state_indices, *, token_indx=None, out=None, out_dtype=None,
                  scale=None, norm_eps=1e-5):
    """Non-speculative single-token in-place update; returns new tensors."""
    return prepare_decode_update(q, k, v, z, a, b, A_log, dt_bias, norm_weight, pool,
                                 state_indices, token_indx=token_indx, out=out,
                                 out_dtype=out_dtype, scale=scale,
                                 norm_eps=norm_eps).run().result()


def prepare_prefill_update(q, k, v, z, a, b, A_log, dt_bias, norm_weight, pool, cu_seqlens,
                           state_indices, *, has_initial_state=None, token_indx=None,
                           chunk_size=64, out=None, out_dtype=None, scale=None,
                           norm_eps=1e-5) -> PreparedCall:
    """prefill_update's arguments marshalled for the C call."""
    arrs, out64, odt, pool64, (n_tok, HK, HV, K, V) = _prepare(
        q, k, v, z, a, b, A_log, dt_bias, norm_weight, pool, out, out_dtype)
    cu = _i32(cu_seqlens)
    si = _i32(state_indices)
    hi = _i32(has_initial_state)
    ti = _i32(token_indx)
    scale = K ** -0.5 if scale is None else scale
    args = (*[_p(x) for x in arrs], _p(out64), _FMT[odt], _p(pool64), _FMT[pool.dtype],
            pool.shape[0], n_tok, _p(cu), cu.shape[0] - 1, _p(si), _p(hi), _p(ti),
            int(chunk_size), HK, HV, K, V, float(scale), float(norm_eps))
    keep = (arrs, cu, si, hi, ti, out64, pool64)
    return PreparedCall("orc_prefill_update", args, keep,
                        "prefill_update", _tensors_back(pool64, pool.dtype, out64, odt))


def prefill_update(q, k, v, z, a, b, A_log, dt_bias, norm_weight, pool, cu_seqlens,
                   state_indices, *, has_initial_state=None, token_indx=None, chunk_size=64,
                   out=None, out_dtype=None, scale=None, norm_eps=1e-5):
    """Chunked prefill: one slot per sequence, the state rounded to the pool
    dtype after every chunk_size-th token and after the last; returns
    ``(pool_after, out_after)`` as new tensors."""
    return prepare_prefill_update(q, k, v, z, a, b, A_log, dt_bias, norm_weight, pool,
                                  cu_seqlens, state_indices,
                                  has_initial_state=has_initial_state, token_indx=token_indx,
                                  chunk_size=chunk_size, out=out, out_dtype=out_dtype,
                                  scale=scale, norm_eps=norm_eps).run().result()


CONV_ACT = {None: 0, "none": 0, "silu": 1}


def _conv_prepare(x, weight, bias, cache, cu, lines, num_acc, token_indx, out, out_dtype,
                  activation, B) -> PreparedCall:
    n_tok, C = x.shape
    num_lines, state_len, C2 = cache.shape
    Cw, width = weight.shape
    assert C2 == C and Cw == C
    if out is None:
        out = torch.zeros((n_tok, C), dtype=out_dtype or x.dtype)
    odt = out.dtype
    x64, w64 = _f64(x), _f64(weight)
    b64 = None if bias is None else _f64(bias)
    out64, cache64 = _f64(out).copy(), _f64(cache).copy()
    args = (_p(x64), _p(out64), _FMT[odt], _p(cache64), _FMT[cache.dtype], num_lines, state_len,
            n_tok, C, width, _p(w64), _p(b64), CONV_ACT[activation], _p(cu), B, _p(lines),
            _p(num_acc), _p(token_indx))
    keep = (x64, w64, b64, cu, lines, num_acc, token_indx, out64, cache64)
    return PreparedCall("orc_conv_update", args, keep,
                        "conv update", _tensors_back(cache64, cache.dtype, out64, odt))


def prepare_conv_spec_update(x, weight, bias, cache, cu_seqlens, conv_indices,
                             num_accepted_tokens, *, token_indx=None, out=None, out_dtype=None,
                             activation="silu") -> PreparedCall:
    """conv_spec_update's arguments marshalled for the C call."""
    cu = _i32(cu_seqlens)
    return _conv_prepare(x, weight, bias, cache, cu, _i32(conv_indices),
                         _i32(num_accepted_tokens), _i32(token_indx), out, out_dtype,
                         activation, cu.shape[0] - 1)


def conv_spec_update(x, weight, bias, cache, cu_seqlens, conv_indices, num_accepted_tokens,
                     *, token_indx=None, out=None, out_dtype=None, activation="silu"):
    """Speculative conv update with rewind; returns ``(cache_after, out_after)``.

    ``x`` is ``[n_tok, C]``, ``weight`` ``[C, width]``, ``cache``
    ``[num_lines, state_len, C]`` (any strides; the result is contiguous).
    ``conv_indices[b]`` is the buffer line of sequence b.  Inputs are not
    modified.
    """
    return prepare_conv_spec_update(x, weight, bias, cache, cu_seqlens, conv_indices,
                                    num_accepted_tokens, token_indx=token_indx, out=out,
                                    out_dtype=out_dtype, activation=activation).run().result()


def conv_decode_update(x, weight, bias, cache, conv_indices, *, token_indx=None, out=None,
                       out_dtype=None, activation="silu"):
    """Non-speculative single-token conv update (a negative line is padding)."""
    lines = _i32(conv_indices)
    return _conv_prepare(x, weight, bias, cache, None, lines, None, _i32(token_indx), out,
                         out_dtype, activation, lines.shape[0]).run().result()
