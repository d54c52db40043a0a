"""Python binding of libgdn_spec.so: argument marshalling only.

Every step of the update runs in the HIP kernels of the library; this module
turns torch device tensors into the C structs of ``include/gdn_spec.h`` and
enqueues on torch's current stream.  Nothing here computes, copies or casts
tensor data, and there is no fallback: a missing library or a non-OK status
raises.

The argument list follows the fused post-conv MTP decode op of vLLM PR #51674
(report section 关键源码片段, the ``fused_gdn_decode_post_conv_mtp`` wrapper:
q/k/v split views, gates a/b, A_log, dt_bias, state indices, cu_seqlens,
num_accepted_tokens, the state pool, output gate z, norm weight, out,
scale = K**-0.5, norm_eps = 1e-5), with the speculative slot table of PR
#46090 and the gather index of PR #51812.  The conv update that precedes it
(``include/gdn_conv.h``) takes the packed projection, the depthwise conv
weight and bias and the wide rolling conv buffer of PR #46090's speculative
path, with the rewind keyed by num_accepted_tokens of PR #51674.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn_spec.so")
ABI_VERSION = 5
MAX_DRAFT_TOKENS = 8

GDN_F32, GDN_F16, GDN_BF16, GDN_F8E4M3 = 0, 1, 2, 3
_DTYPE = {torch.float32: GDN_F32, torch.float16: GDN_F16, torch.bfloat16: GDN_BF16}
_STATE_DTYPE = dict(_DTYPE)
_STATE_DTYPE[torch.float8_e4m3fn] = GDN_F8E4M3
STATUS = {0: "GDN_OK", 1: "GDN_ERR_INVALID", 2: "GDN_ERR_UNSUPPORTED", 3: "GDN_ERR_DEVICE"}


class GdnError(RuntimeError):
    def __init__(self, status: int, reason: str):
        super().__init__(f"{STATUS.get(status, status)}: {reason}")
        self.status = status
        self.reason = reason


class GdnView(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("stride_tok", ctypes.c_int64),
                ("stride_head", ctypes.c_int64)]


class GdnLayer(ctypes.Structure):
    _fields_ = [("q", GdnView), ("k", GdnView), ("v", GdnView), ("z", GdnView),
                ("a", GdnView), ("b", GdnView), ("out", GdnView),
                ("A_log", ctypes.c_void_p), ("dt_bias", ctypes.c_void_p),
                ("norm_weight", ctypes.c_void_p),
                ("act_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("num_k_heads", ctypes.c_int32), ("num_v_heads", ctypes.c_int32),
                ("head_k_dim", ctypes.c_int32), ("head_v_dim", ctypes.c_int32),
                ("n_tok", ctypes.c_int64), ("scale", ctypes.c_float),
                ("norm_eps", ctypes.c_float)]


class GdnStatePool(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("num_slots", ctypes.c_int64)]


class GdnConvLayer(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("x_stride_tok", ctypes.c_int64),
                ("out", ctypes.c_void_p), ("out_stride_tok", ctypes.c_int64),
                ("weight", ctypes.c_void_p), ("bias", ctypes.c_void_p),
                ("x_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("channels", ctypes.c_int32), ("width", ctypes.c_int32),
                ("activation", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("n_tok", ctypes.c_int64)]


class GdnConvCache(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("state_len", ctypes.c_int32), ("num_lines", ctypes.c_int64),
                ("stride_line", ctypes.c_int64), ("stride_pos", ctypes.c_int64),
                ("stride_chan", ctypes.c_int64)]


CONV_MAX_WIDTH = 4
CONV_ACT = {None: 0, "none": 0, "silu": 1}

_lib = None

# Every symbol the header declares, with its ctypes signature.
_VP, _I32, _I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
SIGNATURES = {
    "gdn_spec_decode_update": (ctypes.c_int, [ctypes.POINTER(GdnLayer),
                                              ctypes.POINTER(GdnStatePool), _VP, _I32, _I32,
                                              _VP, _I32, _VP, _VP, _VP]),
    "gdn_decode_update": (ctypes.c_int, [ctypes.POINTER(GdnLayer),
                                         ctypes.POINTER(GdnStatePool), _VP, _I32, _VP, _VP]),
    "gdn_mixed_decode_update": (ctypes.c_int, [ctypes.POINTER(GdnLayer),
                                               ctypes.POINTER(GdnStatePool), _VP, _I32, _I32,
                                               _VP, _I32, _VP, _VP, _VP, _I32, _VP, _VP]),
    "gdn_prefill_update": (ctypes.c_int, [ctypes.POINTER(GdnLayer),
                                          ctypes.POINTER(GdnStatePool), _VP, _I32, _VP, _VP,
                                          _VP, _I32, _VP]),
    "gdn_validate_prefill_indices_host": (ctypes.c_int, [_I64, _I64, _VP, _I32, _VP, _VP]),
    "gdn_validate_indices_host": (ctypes.c_int, [_I64, _I64, _VP, _I32, _I32, _VP, _I32,
                                                 _VP, _VP, _VP, _I32, _VP]),
    "gdn_cast_to_state": (ctypes.c_int, [_VP, _VP, _I64, _I32, _VP]),
    "gdn_last_error": (ctypes.c_char_p, []),
    "gdn_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "gdn_abi_version": (ctypes.c_int32, []),
    "gdn_abi_struct_sizes": (None, [ctypes.POINTER(ctypes.c_size_t)] * 3),
    "gdn_conv_spec_update": (ctypes.c_int, [ctypes.POINTER(GdnConvLayer),
                                            ctypes.POINTER(GdnConvCache), _VP, _I32, _I32,
                                            _VP, _VP, _VP, _VP]),
    "gdn_conv_decode_update": (ctypes.c_int, [ctypes.POINTER(GdnConvLayer),
                                              ctypes.POINTER(GdnConvCache), _VP, _I32, _VP,
                                              _VP]),
    "gdn_validate_conv_indices_host": (ctypes.c_int, [_I64, _I32, _I32, _I64, _VP, _I32, _I32,
                                                      _VP, _VP, _VP, _VP, _I32, _VP]),
    "gdn_conv_abi_struct_sizes": (None, [ctypes.POINTER(ctypes.c_size_t)] * 2),
    "gdn_traffic_pattern": (ctypes.c_int, [ctypes.POINTER(GdnLayer),
                                           ctypes.POINTER(GdnStatePool), _VP, _I32, _I32, _VP,
                                           _I32, _VP, _VP, _VP, _I32, _VP, _I32, _VP]),
    "gdn_issue_probe": (ctypes.c_int, [_VP, _I32, _I32, _I32, _I32, _VP]),
}


def load_library():
    """Load libgdn_spec.so (built in-tree); raise if it is missing or its ABI
    differs from this binding."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; run `python -m speculative_decode_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.gdn_abi_version() != ABI_VERSION:
        raise RuntimeError(f"libgdn_spec ABI {lib.gdn_abi_version()} != binding {ABI_VERSION}")
    sizes = [ctypes.c_size_t() for _ in range(3)]
    lib.gdn_abi_struct_sizes(*[ctypes.byref(s) for s in sizes])
    want = [ctypes.sizeof(GdnView), ctypes.sizeof(GdnLayer), ctypes.sizeof(GdnStatePool)]
    csizes = [ctypes.c_size_t() for _ in range(2)]
    lib.gdn_conv_abi_struct_sizes(*[ctypes.byref(s) for s in csizes])
    sizes += csizes
    want += [ctypes.sizeof(GdnConvLayer), ctypes.sizeof(GdnConvCache)]
    if [s.value for s in sizes] != want:
        raise RuntimeError(f"struct layout mismatch: library {[s.value for s in sizes]}, "
                           f"binding {want}")
    _lib = lib
    return lib


def last_error() -> str:
    return load_library().gdn_last_error().decode()


def _check(status: int):
    if status != 0:
        raise GdnError(status, last_error())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _view3(t: torch.Tensor, name: str) -> GdnView:
    if t.dim() != 3:
        raise ValueError(f"{name} must be [n_tok, heads, dim]")
    if t.numel() == 0:          # no rows: strides are meaningless
        return GdnView(None, 0, 0)
    if t.stride(-1) != 1:
        raise ValueError(f"{name} must have a contiguous last dim")
    return GdnView(t.data_ptr(), t.stride(0), t.stride(1))


def _view2(t: torch.Tensor, name: str) -> GdnView:
    if t.dim() != 2:
        raise ValueError(f"{name} must be [n_tok, heads]")
    if t.numel() == 0:
        return GdnView(None, 0, 1)
    if t.stride(-1) != 1:
        raise ValueError(f"{name} must have a contiguous last dim")
    return GdnView(t.data_ptr(), t.stride(0), 1)


def _meta(t: Optional[torch.Tensor], name: str, device) -> Optional[torch.Tensor]:
    if t is None:
        return None
    if t.dtype != torch.int32 or not t.is_contiguous() or t.device != device:
        raise ValueError(f"{name} must be a contiguous int32 tensor on {device}")
    return t


def _check_gather(tix: Optional[torch.Tensor], slots: torch.Tensor, tname: str, sname: str):
    """Entry i of a single-token launch reads tix[i]: the gather index needs
    an entry for every slot entry."""
    if tix is not None and tix.numel() < slots.numel():
        raise ValueError(f"{tname} has {tix.numel()} entries, {sname} {slots.numel()}")


def make_layer(q, k, v, z, a, b, A_log, dt_bias, norm_weight, out, *, scale=None,
               norm_eps=1e-5) -> GdnLayer:
    """Describe one layer's device tensors as a gdn_layer (no data is touched)."""
    dev = q.device
    for name, t in (("k", k), ("v", v), ("z", z), ("a", a), ("b", b), ("A_log", A_log),
                    ("dt_bias", dt_bias), ("norm_weight", norm_weight), ("out", out)):
        if t.device != dev:
            raise ValueError(f"{name} is on {t.device}, q on {dev}")
    if not (q.dtype == k.dtype == v.dtype == z.dtype == a.dtype == b.dtype):
        raise ValueError("q, k, v, z, a, b must share one dtype")
    for name, t in (("A_log", A_log), ("dt_bias", dt_bias), ("norm_weight", norm_weight)):
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 tensor")
    if q.dtype not in _DTYPE or out.dtype not in _DTYPE:
        raise ValueError("activations and out must be float32, float16 or bfloat16")
    n_tok, HK, K = q.shape
    HV, V = v.shape[1], v.shape[2]
    for name, t, shp in (("k", k, (n_tok, HK, K)), ("v", v, (n_tok, HV, V)),
                         ("z", z, (n_tok, HV, V)), ("out", out, (n_tok, HV, V)),
                         ("a", a, (n_tok, HV)), ("b", b, (n_tok, HV))):
        if tuple(t.shape) != shp:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shp}")
    return GdnLayer(
        _view3(q, "q"), _view3(k, "k"), _view3(v, "v"), _view3(z, "z"),
        _view2(a, "a"), _view2(b, "b"), _view3(out, "out"),
        A_log.data_ptr(), dt_bias.data_ptr(), norm_weight.data_ptr(),
        _DTYPE[q.dtype], _DTYPE[out.dtype], HK, HV, K, V, n_tok,
        float(K ** -0.5 if scale is None else scale), float(norm_eps))


def make_pool(state: torch.Tensor, layer: Optional[GdnLayer] = None,
              device=None) -> GdnStatePool:
    """Describe a state pool.  With ``layer``, its [HV, V, K] must be the
    layer's: the kernels address tile (slot, h) as slot * HV + h with the
    layer's HV, so a pool with fewer heads would be written past its end."""
    if state.dtype not in _STATE_DTYPE:
        raise ValueError("state pool must be float32, float16, bfloat16 or float8_e4m3fn")
    if state.dim() != 4 or not state.is_contiguous():
        raise ValueError("state pool must be a contiguous [num_slots, HV, V, K] tensor")
    if layer is not None:
        want = (layer.num_v_heads, layer.head_v_dim, layer.head_k_dim)
        if tuple(state.shape[1:]) != want:
            raise ValueError(f"state pool is [num_slots, {', '.join(map(str, state.shape[1:]))}]"
                             f", the layer needs [num_slots, {', '.join(map(str, want))}]")
    if device is not None and state.device != device:
        raise ValueError(f"state pool is on {state.device}, the layer on {device}")
    return GdnStatePool(state.data_ptr(), _STATE_DTYPE[state.dtype], 0, state.shape[0])


def cast_to_state(src: torch.Tensor, dtype: torch.dtype) -> torch.Tensor:
    """fp32 device tensor -> a new tensor in a state format, rounded by the
    library's store conversion (gdn_cast_to_state)."""
    lib = load_library()
    if src.dtype != torch.float32 or not src.is_contiguous():
        raise ValueError("src must be a contiguous float32 tensor")
    if dtype not in _STATE_DTYPE:
        raise ValueError(f"{dtype} is not a state format")
    dst = torch.empty(src.shape, dtype=dtype, device=src.device)
    _check(lib.gdn_cast_to_state(_ptr(src), _ptr(dst), src.numel(), _STATE_DTYPE[dtype],
                                 _stream(src.device)))
    return dst


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def spec_decode_update(q, k, v, z, a, b, A_log, dt_bias, norm_weight, state,
                       cu_seqlens, spec_state_indices, num_accepted_tokens, *,
                       token_indx=None, out=None, scale=None, norm_eps=1e-5,
                       max_q_len=MAX_DRAFT_TOKENS):
    """Speculative update of ``state`` in place; returns ``out``.

    ``spec_state_indices`` is ``[num_seqs, spec_stride]``.  ``out`` defaults to
    ``torch.zeros_like(z)``: only processed rows are written.
    """
    lib = load_library()
    if out is None:
        out = torch.zeros_like(z)
    dev = q.device
    layer = make_layer(q, k, v, z, a, b, A_log, dt_bias, norm_weight, out,
                       scale=scale, norm_eps=norm_eps)
    pool = make_pool(state, layer, dev)
    cu = _meta(cu_seqlens, "cu_seqlens", dev)
    si = _meta(spec_state_indices, "spec_state_indices", dev)
    na = _meta(num_accepted_tokens, "num_accepted_tokens", dev)
    ti = _meta(token_indx, "token_indx", dev)
    if si.dim() != 2:
        raise ValueError("spec_state_indices must be [num_seqs, spec_stride]")
    B = cu.shape[0] - 1
    if si.shape[0] != B or na.shape[0] != B:
        raise ValueError("cu_seqlens, spec_state_indices, num_accepted_tokens disagree on B")
    _check(lib.gdn_spec_decode_update(ctypes.byref(layer), ctypes.byref(pool), _ptr(cu), B,
                                      int(max_q_len), _ptr(si), si.shape[1], _ptr(na),
                                      _ptr(ti), _stream(dev)))
    return out


def decode_update(q, k, v, z, a, b, A_log, dt_bias, norm_weight, state, state_indices, *,
                  token_indx=None, out=None, scale=None, norm_eps=1e-5):
    """Non-speculative single-token update, in place at ``state_indices[i]``
    (negative = padding); returns ``out`` (default zeros)."""
    lib = load_library()
    if out is None:
        out = torch.zeros_like(z)
    dev = q.device
    layer = make_layer(q, k, v, z, a, b, A_log, dt_bias, norm_weight, out,
                       scale=scale, norm_eps=norm_eps)
    pool = make_pool(state, layer, dev)
    si = _meta(state_indices, "state_indices", dev)
    ti = _meta(token_indx, "token_indx", dev)
    _check_gather(ti, si, "token_indx", "state_indices")
    _check(lib.gdn_decode_update(ctypes.byref(layer), ctypes.byref(pool), _ptr(si),
                                 si.shape[0], _ptr(ti), _stream(dev)))
    return out


def mixed_decode_update(q, k, v, z, a, b, A_log, dt_bias, norm_weight, state, cu_seqlens,
                        spec_state_indices, num_accepted_tokens, state_indices, *,
                        spec_token_indx=None, non_spec_token_indx=None, out=None, scale=None,
                        norm_eps=1e-5, max_q_len=MAX_DRAFT_TOKENS):
    """A mixed batch -- speculative sequences and single-token entries -- in
    one launch; returns ``out`` (default zeros)."""
    lib = load_library()
    if out is None:
        out = torch.zeros_like(z)
    dev = q.device
    layer = make_layer(q, k, v, z, a, b, A_log, dt_bias, norm_weight, out,
                       scale=scale, norm_eps=norm_eps)
    pool = make_pool(state, layer, dev)
    cu = _meta(cu_seqlens, "cu_seqlens", dev)
    si = _meta(spec_state_indices, "spec_state_indices", dev)
    na = _meta(num_accepted_tokens, "num_accepted_tokens", dev)
    st = _meta(spec_token_indx, "spec_token_indx", dev)
    ns = _meta(state_indices, "state_indices", dev)
    nst = _meta(non_spec_token_indx, "non_spec_token_indx", dev)
    _check_gather(nst, ns, "non_spec_token_indx", "state_indices")
    if si.dim() != 2:
        raise ValueError("spec_state_indices must be [num_seqs, spec_stride]")
    B = cu.shape[0] - 1
    if si.shape[0] != B or na.shape[0] != B:
        raise ValueError("cu_seqlens, spec_state_indices, num_accepted_tokens disagree on B")
    _check(lib.gdn_mixed_decode_update(ctypes.byref(layer), ctypes.byref(pool), _ptr(cu), B,
                                       int(max_q_len), _ptr(si), si.shape[1], _ptr(na),
                                       _ptr(st), _ptr(ns), ns.shape[0], _ptr(nst),
                                       _stream(dev)))
    return out


def forward_core(q, k, v, z, a, b, A_log, dt_bias, norm_weight, state, *,
                 spec_cu_seqlens=None, spec_state_indices=None, num_accepted_tokens=None,
                 spec_token_indx=None, non_spec_state_indices=None,
                 non_spec_token_indx=None, out=None, scale=None, norm_eps=1e-5,
                 max_q_len=MAX_DRAFT_TOKENS, single_launch=True):
    """Spec / non-spec split of one batch (vLLM PR #51812, ``_forward_core``).

    A pure speculative batch passes ``spec_token_indx=None`` and runs one
    launch with no gather.  A mixed batch gathers the spec rows (q/k/v/z *and*
    the gates a/b, with the same index) and the non-spec rows inside the
    kernel; with ``single_launch`` (the default) both parts run in one launch
    (``gdn_mixed_decode_update``), otherwise as a spec launch followed by a
    single-token launch.  Either way each part writes its own rows of one
    ``out``.
    """
    if out is None:
        out = torch.zeros_like(z)
    has_spec = spec_cu_seqlens is not None and spec_cu_seqlens.shape[0] > 1
    has_ns = non_spec_state_indices is not None and non_spec_state_indices.shape[0] > 0
    if single_launch and has_spec and has_ns:
        return mixed_decode_update(q, k, v, z, a, b, A_log, dt_bias, norm_weight, state,
                                   spec_cu_seqlens, spec_state_indices, num_accepted_tokens,
                                   non_spec_state_indices, spec_token_indx=spec_token_indx,
                                   non_spec_token_indx=non_spec_token_indx, out=out,
                                   scale=scale, norm_eps=norm_eps, max_q_len=max_q_len)
    if has_spec:
        spec_decode_update(q, k, v, z, a, b, A_log, dt_bias, norm_weight, state,
                           spec_cu_seqlens, spec_state_indices, num_accepted_tokens,
                           token_indx=spec_token_indx, out=out, scale=scale,
                           norm_eps=norm_eps, max_q_len=max_q_len)
    if has_ns:
        decode_update(q, k, v, z, a, b, A_log, dt_bias, norm_weight, state,
                      non_spec_state_indices, token_indx=non_spec_token_indx, out=out,
                      scale=scale, norm_eps=norm_eps)
    return out


def traffic_pattern(q, k, v, z, a, b, A_log, dt_bias, norm_weight, state, *,
                    spec_cu_seqlens=None, spec_state_indices=None, num_accepted_tokens=None,
                    spec_token_indx=None, non_spec_state_indices=None,
                    non_spec_token_indx=None, out=None, scale=None, norm_eps=1e-5,
                    max_q_len=MAX_DRAFT_TOKENS, single_launch=True, blocks_per_cu=0):
    """The HBM traffic of the forward_core launch with the same arguments and
    no arithmetic (gdn_traffic_pattern, include/gdn_bench.h): a measurement
    of the memory system's ceiling for that traffic.  Overwrites the written
    slots of ``state`` with copies of the rewind tiles and ``out`` with
    meaningless bits.  ``single_launch`` is accepted for symmetry with
    forward_core; a mixed batch is always one launch here.  ``blocks_per_cu``
    > 0 replaces the kernel's blocks per CU."""
    lib = load_library()
    if out is None:
        out = torch.zeros_like(z)
    dev = q.device
    layer = make_layer(q, k, v, z, a, b, A_log, dt_bias, norm_weight, out,
                       scale=scale, norm_eps=norm_eps)
    pool = make_pool(state, layer, dev)
    has_spec = spec_cu_seqlens is not None and spec_cu_seqlens.shape[0] > 1
    cu = _meta(spec_cu_seqlens, "cu_seqlens", dev) if has_spec else None
    si = _meta(spec_state_indices, "spec_state_indices", dev) if has_spec else None
    na = _meta(num_accepted_tokens, "num_accepted_tokens", dev) if has_spec else None
    st = _meta(spec_token_indx, "spec_token_indx", dev) if has_spec else None
    ns = _meta(non_spec_state_indices, "state_indices", dev)
    nst = _meta(non_spec_token_indx, "non_spec_token_indx", dev)
    B = cu.shape[0] - 1 if has_spec else 0
    _check(lib.gdn_traffic_pattern(ctypes.byref(layer), ctypes.byref(pool), _ptr(cu), B,
                                   int(max_q_len), _ptr(si), si.shape[1] if has_spec else 1,
                                   _ptr(na), _ptr(st), _ptr(ns),
                                   0 if ns is None else ns.shape[0], _ptr(nst),
                                   int(blocks_per_cu), _stream(dev)))
    return out


def issue_probe(out: torch.Tensor, mode: int, n_mfma: int, n_valu: int):
    """One launch of the FP32 matrix / vector issue probe (gdn_issue_probe,
    include/gdn_bench.h) with out.numel() // 512 blocks of 512 threads."""
    lib = load_library()
    if out.dtype != torch.float32 or not out.is_contiguous() or out.numel() % 512:
        raise ValueError("out must be a contiguous float32 tensor of blocks * 512 elements")
    _check(lib.gdn_issue_probe(_ptr(out), out.numel() // 512, mode, n_mfma, n_valu,
                               _stream(out.device)))


def prefill_update(q, k, v, z, a, b, A_log, dt_bias, norm_weight, state, cu_seqlens,
                   state_indices, *, has_initial_state=None, token_indx=None, out=None,
                   chunk_size=64, scale=None, norm_eps=1e-5):
    """Chunked prefill of ``state`` in place (one slot per sequence, the state
    rounded to its dtype every ``chunk_size`` rows); returns ``out`` (default
    zeros)."""
    lib = load_library()
    if out is None:
        out = torch.zeros_like(z)
    dev = q.device
    layer = make_layer(q, k, v, z, a, b, A_log, dt_bias, norm_weight, out,
                       scale=scale, norm_eps=norm_eps)
    pool = make_pool(state, layer, dev)
    cu = _meta(cu_seqlens, "cu_seqlens", dev)
    si = _meta(state_indices, "state_indices", dev)
    hi = _meta(has_initial_state, "has_initial_state", dev)
    ti = _meta(token_indx, "token_indx", dev)
    B = cu.shape[0] - 1
    if si.shape[0] != B or (hi is not None and hi.shape[0] != B):
        raise ValueError("cu_seqlens, state_indices, has_initial_state disagree on B")
    _check(lib.gdn_prefill_update(ctypes.byref(layer), ctypes.byref(pool), _ptr(cu), B, _ptr(si),
                                  _ptr(hi), _ptr(ti), int(chunk_size), _stream(dev)))
    return out


def validate_prefill_indices(num_slots: int, n_tok: int, cu_seqlens, state_indices, *,
                             token_indx=None):
    """Check prefill metadata on host copies (gdn_validate_prefill_indices_host)."""
    lib = load_library()

    def host(t):
        return None if t is None else t.detach().to("cpu", torch.int32).contiguous()

    cu, si, ti = host(cu_seqlens), host(state_indices), host(token_indx)
    _check(lib.gdn_validate_prefill_indices_host(int(num_slots), int(n_tok), _ptr(cu),
                                                 cu.shape[0] - 1, _ptr(si), _ptr(ti)))


def prefill_batch_args(batch, device, *, state=None, out=None):
    """Device copies of a workloads.PrefillBatch as keyword arguments of
    prefill_update."""
    def d(t):
        return None if t is None else t.to(device)
    return dict(q=d(batch.q), k=d(batch.k), v=d(batch.v), z=d(batch.z), a=d(batch.a),
                b=d(batch.b), A_log=d(batch.A_log), dt_bias=d(batch.dt_bias),
                norm_weight=d(batch.norm_weight),
                state=d(batch.pool) if state is None else state,
                cu_seqlens=d(batch.cu_seqlens), state_indices=d(batch.state_indices),
                has_initial_state=d(batch.has_initial_state), token_indx=d(batch.token_indx),
                out=out, chunk_size=batch.chunk_size, scale=batch.scale,
                norm_eps=batch.norm_eps)


def validate_indices(num_slots: int, n_tok: int, *, cu_seqlens=None, spec_state_indices=None,
                     num_accepted_tokens=None, spec_token_indx=None, state_indices=None,
                     non_spec_token_indx=None, max_q_len=MAX_DRAFT_TOKENS):
    """Check the metadata contract on host copies (gdn_validate_indices_host).
    Raises GdnError with the first violation."""
    lib = load_library()

    def host(t):
        return None if t is None else t.detach().to("cpu", torch.int32).contiguous()

    cu, si, na = host(cu_seqlens), host(spec_state_indices), host(num_accepted_tokens)
    st, ns, nst = host(spec_token_indx), host(state_indices), host(non_spec_token_indx)
    B = 0 if cu is None else cu.shape[0] - 1
    stride = 1 if si is None else (si.shape[1] if si.dim() == 2 else 1)
    _check(lib.gdn_validate_indices_host(
        int(num_slots), int(n_tok), _ptr(cu), B, int(max_q_len), _ptr(si), stride, _ptr(na),
        _ptr(st), _ptr(ns), 0 if ns is None else ns.shape[0], _ptr(nst)))


def batch_args(batch, device, *, state=None, out=None):
    """Device copies of a workloads.GDNBatch as keyword arguments of
    forward_core (convenience for tests and the benchmark)."""
    def d(t):
        return None if t is None else t.to(device)
    return dict(q=d(batch.q), k=d(batch.k), v=d(batch.v), z=d(batch.z), a=d(batch.a),
                b=d(batch.b), A_log=d(batch.A_log), dt_bias=d(batch.dt_bias),
                norm_weight=d(batch.norm_weight),
                state=d(batch.pool) if state is None else state,
                spec_cu_seqlens=d(batch.cu_seqlens),
                spec_state_indices=d(batch.spec_state_indices),
                num_accepted_tokens=d(batch.num_accepted_tokens),
                spec_token_indx=d(batch.spec_token_indx),
                non_spec_state_indices=d(batch.state_indices),
                non_spec_token_indx=d(batch.non_spec_token_indx),
                out=out, scale=batch.scale, norm_eps=batch.norm_eps,
                max_q_len=max(1, batch.T))


# ---- conv update with rewind (include/gdn_conv.h) ---------------------------
def make_conv_layer(x, weight, bias, out, *, activation="silu") -> GdnConvLayer:
    """Describe the conv inputs ``x`` [n_tok, C], the depthwise ``weight``
    [C, width] (or torch's [C, 1, width]), ``bias`` [C] or None and ``out``
    [n_tok, C] as a gdn_conv_layer (no data is touched)."""
    if weight.dim() == 3 and weight.shape[1] == 1:
        weight = weight[:, 0, :]
    if x.dim() != 2 or out.dim() != 2 or tuple(out.shape) != tuple(x.shape):
        raise ValueError("x and out must both be [n_tok, channels]")
    n_tok, C = x.shape
    if weight.dim() != 2 or weight.shape[0] != C:
        raise ValueError(f"weight must be [channels={C}, width]")
    if weight.dtype != torch.float32 or not weight.is_contiguous():
        raise ValueError("weight must be a contiguous float32 tensor")
    if bias is not None and (bias.dtype != torch.float32 or not bias.is_contiguous()
                             or tuple(bias.shape) != (C,)):
        raise ValueError("bias must be a contiguous float32 [channels] tensor or None")
    if x.dtype not in _DTYPE or out.dtype not in _DTYPE:
        raise ValueError("x and out must be float32, float16 or bfloat16")
    for name, t in (("weight", weight), ("bias", bias), ("out", out)):
        if t is not None and t.device != x.device:
            raise ValueError(f"{name} is on {t.device}, x on {x.device}")
    if activation not in CONV_ACT:
        raise ValueError(f"activation must be one of {sorted(k for k in CONV_ACT if k)}")
    empty = x.numel() == 0
    if not empty and (x.stride(-1) != 1 or out.stride(-1) != 1):
        raise ValueError("x and out must have a contiguous channel dim")
    return GdnConvLayer(
        None if empty else x.data_ptr(), 0 if empty else x.stride(0),
        None if empty else out.data_ptr(), C if empty else out.stride(0),
        weight.data_ptr(), None if bias is None else bias.data_ptr(),
        _DTYPE[x.dtype], _DTYPE[out.dtype], C, weight.shape[1], CONV_ACT[activation], 0, n_tok)


def make_conv_cache(cache: torch.Tensor, layer: Optional[GdnConvLayer] = None,
                    device=None) -> GdnConvCache:
    """A [num_lines, state_len, C] buffer with any strides (a channel-major
    buffer is passed as ``buf.transpose(1, 2)``).  With ``layer``, C must be
    the layer's channel count: the kernels index every channel of a line."""
    if cache.dim() != 3 or cache.dtype not in _DTYPE:
        raise ValueError("conv cache must be a float32/float16/bfloat16 "
                         "[num_lines, state_len, channels] tensor")
    if layer is not None and cache.shape[2] != layer.channels:
        raise ValueError(f"conv cache has {cache.shape[2]} channels, the layer "
                         f"{layer.channels}")
    if device is not None and cache.device != device:
        raise ValueError(f"conv cache is on {cache.device}, x on {device}")
    return GdnConvCache(cache.data_ptr(), _DTYPE[cache.dtype], cache.shape[1], cache.shape[0],
                        cache.stride(0), cache.stride(1), cache.stride(2))


def _conv_weight(weight):
    return weight[:, 0, :] if weight.dim() == 3 and weight.shape[1] == 1 else weight


def conv_spec_update(x, weight, bias, cache, cu_seqlens, conv_indices, num_accepted_tokens, *,
                     token_indx=None, out=None, activation="silu",
                     max_q_len=MAX_DRAFT_TOKENS):
    """Speculative conv update of ``cache`` in place with rewind; returns
    ``out`` (default zeros shaped like ``x``; only processed rows are written)."""
    lib = load_library()
    if out is None:
        out = torch.zeros_like(x)
    dev = x.device
    layer = make_conv_layer(x, _conv_weight(weight), bias, out, activation=activation)
    cc = make_conv_cache(cache, layer, dev)
    cu = _meta(cu_seqlens, "cu_seqlens", dev)
    li = _meta(conv_indices, "conv_indices", dev)
    na = _meta(num_accepted_tokens, "num_accepted_tokens", dev)
    ti = _meta(token_indx, "token_indx", dev)
    B = cu.shape[0] - 1
    if li.shape[0] != B or na.shape[0] != B:
        raise ValueError("cu_seqlens, conv_indices, num_accepted_tokens disagree on B")
    _check(lib.gdn_conv_spec_update(ctypes.byref(layer), ctypes.byref(cc), _ptr(cu), B,
                                    int(max_q_len), _ptr(li), _ptr(na), _ptr(ti), _stream(dev)))
    return out


def conv_decode_update(x, weight, bias, cache, conv_indices, *, token_indx=None, out=None,
                       activation="silu"):
    """Non-speculative single-token conv update at line ``conv_indices[i]``
    (negative = padding); returns ``out`` (default zeros)."""
    lib = load_library()
    if out is None:
        out = torch.zeros_like(x)
    dev = x.device
    layer = make_conv_layer(x, _conv_weight(weight), bias, out, activation=activation)
    cc = make_conv_cache(cache, layer, dev)
    li = _meta(conv_indices, "conv_indices", dev)
    ti = _meta(token_indx, "token_indx", dev)
    _check_gather(ti, li, "token_indx", "conv_indices")
    _check(lib.gdn_conv_decode_update(ctypes.byref(layer), ctypes.byref(cc), _ptr(li),
                                      li.shape[0], _ptr(ti), _stream(dev)))
    return out


def validate_conv_indices(num_lines: int, state_len: int, width: int, n_tok: int, *,
                          cu_seqlens=None, conv_indices=None, num_accepted_tokens=None,
                          spec_token_indx=None, decode_indices=None, decode_token_indx=None,
                          max_q_len=MAX_DRAFT_TOKENS):
    """Check the conv metadata contract on host copies
    (gdn_validate_conv_indices_host).  Raises GdnError with the first violation."""
    lib = load_library()

    def host(t):
        return None if t is None else t.detach().to("cpu", torch.int32).contiguous()

    cu, li, na = host(cu_seqlens), host(conv_indices), host(num_accepted_tokens)
    st, dl, dt = host(spec_token_indx), host(decode_indices), host(decode_token_indx)
    B = 0 if cu is None else cu.shape[0] - 1
    _check(lib.gdn_validate_conv_indices_host(
        int(num_lines), int(state_len), int(width), int(n_tok), _ptr(cu), B, int(max_q_len),
        _ptr(li), _ptr(na), _ptr(st), _ptr(dl), 0 if dl is None else dl.shape[0], _ptr(dt)))


def conv_batch_args(batch, device, *, cache=None, out=None):
    """Device copies of a workloads.ConvBatch as keyword arguments of
    conv_spec_update (convenience for tests and the benchmark)."""
    def d(t):
        return None if t is None else t.to(device)
    return dict(x=d(batch.x), weight=d(batch.weight), bias=d(batch.bias),
                cache=d(batch.cache) if cache is None else cache,
                cu_seqlens=d(batch.cu_seqlens), conv_indices=d(batch.conv_indices),
                num_accepted_tokens=d(batch.num_accepted_tokens),
                token_indx=d(batch.token_indx), out=out, activation=batch.activation,
                max_q_len=max(1, batch.T))
